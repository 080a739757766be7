// Replays a validation matrix through the C ABI (include/fa.h) in a process
// built with the host address and undefined-behaviour sanitizers.
//
// stdin: one case per line, "<entry> <expected status> <hex bytes of the
// parameter struct>", where entry is one of
//   fwd bwd stage0 stage1 stage2 bwd_ws bwd_na kv kv_ws vl_fwd vl_bwd vl_ws
// (stageN: fa_bwd_stage N; bwd_na: fa_bwd_noalloc)
// Pointer arguments are fixed, distinct, 16-byte aligned fake addresses: the
// ABI validates them and never dereferences one before its device check.
// Prints every mismatch; the exit status is the number of mismatches (capped).
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "fa.h"

namespace {

void* P(unsigned i) { return reinterpret_cast<void*>(static_cast<uintptr_t>(0x10000u * (i + 1))); }

bool from_hex(const char* hex, std::vector<unsigned char>& out) {
  const size_t n = std::strlen(hex);
  if (n % 2) return false;
  out.resize(n / 2);
  for (size_t i = 0; i < n / 2; ++i) {
    unsigned v = 0;
    if (std::sscanf(hex + 2 * i, "%2x", &v) != 1) return false;
    out[i] = static_cast<unsigned char>(v);
  }
  return true;
}

int run(const std::string& entry, const std::vector<unsigned char>& bytes, bool* known) {
  *known = true;
  size_t ws = 0;
  const size_t big = size_t(1) << 30;
  if (entry == "fwd" || entry == "bwd" || entry == "bwd_ws" || entry == "bwd_na" || entry.rfind("stage", 0) == 0) {
    if (bytes.size() != sizeof(fa_params)) return -100;
    fa_params p;
    std::memcpy(&p, bytes.data(), sizeof p);
    if (entry == "fwd") return fa_fwd(&p, P(0), P(1), P(2), P(3), static_cast<float*>(P(4)), nullptr);
    if (entry == "bwd")
      return fa_bwd(&p, P(9), P(0), P(1), P(2), P(3), static_cast<float*>(P(4)), P(6), P(7), P(8), P(5), big,
                    nullptr);
    if (entry == "bwd_ws") return fa_bwd_workspace_size(&p, &ws);
    if (entry == "bwd_na")
      return fa_bwd_noalloc(&p, P(9), P(0), P(1), P(2), P(3), static_cast<float*>(P(4)), P(6), P(7), P(8), nullptr);
    const int st = entry[5] - '0';
    return fa_bwd_stage(&p, st, P(9), P(0), P(1), P(2), P(3), static_cast<float*>(P(4)), P(6), P(7), P(8), P(5),
                        big, nullptr);
  }
  if (entry == "kv" || entry == "kv_ws") {
    if (bytes.size() != sizeof(fa_kvcache_params)) return -100;
    fa_kvcache_params p;
    std::memcpy(&p, bytes.data(), sizeof p);
    if (entry == "kv_ws") return fa_fwd_kvcache_workspace_size(&p, &ws);
    return fa_fwd_kvcache(&p, P(20), P(21), P(22), static_cast<const int32_t*>(P(23)), P(24), P(25), P(26),
                          static_cast<float*>(P(27)), P(28), big, nullptr);
  }
  if (entry == "vl_fwd" || entry == "vl_bwd" || entry == "vl_ws") {
    if (bytes.size() != sizeof(fa_varlen_params)) return -100;
    fa_varlen_params p;
    std::memcpy(&p, bytes.data(), sizeof p);
    const int32_t* cq = static_cast<const int32_t*>(P(40));
    const int32_t* ck = static_cast<const int32_t*>(P(41));
    if (entry == "vl_ws") return fa_bwd_varlen_workspace_size(&p, &ws);
    if (entry == "vl_fwd") return fa_fwd_varlen(&p, P(0), P(1), P(2), cq, ck, P(3), static_cast<float*>(P(4)), nullptr);
    return fa_bwd_varlen(&p, P(9), P(0), P(1), P(2), P(3), static_cast<float*>(P(4)), cq, ck, P(6), P(7), P(8), P(5),
                         big, nullptr);
  }
  *known = false;
  return -1;
}

}  // namespace

int main() {
  int bad = 0, cases = 0;
  char entry[32], hex[8192];
  int expected = 0;
  while (std::scanf("%31s %d %8191s", entry, &expected, hex) == 3) {
    std::vector<unsigned char> bytes;
    if (!from_hex(hex, bytes)) {
      std::printf("malformed case %d\n", cases);
      ++bad;
      continue;
    }
    bool known = false;
    const int got = run(entry, bytes, &known);
    ++cases;
    if (!known || got != expected) {
      std::printf("case %d %s: expected %d got %d (%s)\n", cases, entry, expected, got, fa_last_error());
      ++bad;
    } else if (got != FA_OK && fa_last_error()[0] == '\0') {
      std::printf("case %d %s: status %d without a message\n", cases, entry, got);
      ++bad;
    }
  }
  // Calls with no parameter struct, and the constant-returning functions.
  if (fa_fwd(nullptr, P(0), P(1), P(2), P(3), static_cast<float*>(P(4)), nullptr) != FA_ERR_INVALID_ARG) ++bad;
  if (fa_fwd_kvcache(nullptr, P(0), P(1), P(2), nullptr, nullptr, nullptr, P(3), nullptr, nullptr, 0, nullptr) !=
      FA_ERR_INVALID_ARG)
    ++bad;
  for (int s = 0; s <= 4; ++s)
    if (!fa_status_string(static_cast<fa_status>(s))[0]) ++bad;
  if (fa_version() != FA_VERSION) ++bad;
  std::printf("%d cases, %d mismatches\n", cases, bad);
  return bad > 100 ? 100 : bad;
}
