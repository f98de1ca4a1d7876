// State shared by the launch stand-ins and the host driver (sanitizer build).
#pragma once
#include <stddef.h>

struct StubState {
  const void* ws = nullptr;  // the workspace of the current call
  size_t ws_bytes = 0;
  bool user_mass = false;    // the caller passed its own block-mass buffer
  bool user_kbar = false;    // the caller passed its own pooled keys (decode)
  bool fail_launch = false;  // make the first launch report a failure
  long calls = 0;
  long batched_launches = 0;  // head-pair attention launches over several sequences
  long batched_items = 0;
  long single_launches = 0;   // attention launches over one sequence
  long batched_searches = 0;  // search-stage launches over several sequences
};
extern StubState g_stub;
