// stub_state.h - what the host-only launcher stubs (hip_stub.cpp) record.
// Test infrastructure only.
#pragma once

#include "fa_internal.h"

struct StubState {
  enum Kind { NONE, FWD, FWD_PAGED, DECODE, CASCADE, APPEND, BWD };
  int launches = 0;
  int copies = 0;
  int scratch_lookups = 0;
  bool fail_copies = false;  // make hipMemcpyAsync report an error
  Kind last_kind = NONE;
  int grid = 0;
  fa::FwdParams fwd{};
  fa::DecodeParams dec{};
  fa::AppendParams app{};
  fa::BwdParams bwd{};
};

extern StubState g_stub;
