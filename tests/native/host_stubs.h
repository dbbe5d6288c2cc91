// What the stand-in launchers of host_stubs.cpp recorded (test infrastructure).
#pragma once

#include "attn_internal.h"

struct StubRecord {
  attn::PrefillArgs prefill{};
  attn::PagedArgs paged{};
  attn::AppendArgs append{};
  attn::NormArgs norm{};
  int prefill_bf16 = 0, prefill_f32 = 0, paged_prefill = 0, paged_decode = 0, append_calls = 0,
      norm_calls = 0, scratch_lookups = 0;
};

extern StubRecord g_stub;
constexpr uintptr_t kStubScratchAddress = 0x7f0000000000ull;
