// Host-side choice of the GEMM kernel and its tile from the problem shape
// and the device's CU count. Plain C++, no HIP types, so the rules also
// compile and can be checked on a host without a GPU; the launchers in
// gemm.hip map each answer onto a template instance.

#pragma once

#include <stdint.h>

namespace w8a8 {
namespace dispatch {

constexpr int kMidBK = 128;       // K bytes per stage of the LDS-staged kernels
constexpr int kSkinnyMaxM = 64;   // one M tile of the decode kernels covers the tokens
constexpr int kPrefillMinM = 512; // other K: the 64-byte-stage prefill kernel from here

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Which M take the LDS-staged decode kernel (K % 128 == 0): every decode M,
// and beyond that while M tiles of 64 rows beat the prefill kernel's 256-row
// tiles, which fill the 256 CUs only once there are enough of them (measured
// on MI355X, Llama-3.1-8B shapes: up to M = 128 for 28672 channels, 1536 for
// K = 14336, 1024 otherwise).
inline bool mid_path(int64_t M, int64_t N, int64_t K) {
  if (K % kMidBK != 0) return false;
  if (M <= kSkinnyMaxM) return true;
  if (N >= 16384) return M <= 128;
  return M <= (K > 8192 ? 1536 : 1024);
}

enum class GemmPath {
  kMid,         // LDS-staged decode kernel, K % 128 == 0 (also M-tiled past 64)
  kSkinny,      // register-staged decode kernel, other K, M <= 64
  kPrefill128,  // full-line prefill kernel, K % 128 == 0
  kPrefill64,   // 64-byte-stage prefill kernel, other K, M >= 512
  kTiled,       // register-staged 128 x 128 tiles, other K, 64 < M < 512
};

inline GemmPath gemm_path(int64_t M, int64_t N, int64_t K) {
  if (mid_path(M, N, K)) return GemmPath::kMid;
  if (M <= kSkinnyMaxM) return GemmPath::kSkinny;
  if (K % kMidBK == 0) return GemmPath::kPrefill128;
  return M >= kPrefillMinM ? GemmPath::kPrefill64 : GemmPath::kTiled;
}

// Template arguments of the decode kernel: 16 * mt token rows and 16 * rw
// output channels per workgroup, nw waves, ns-stage LDS ring per wave.
struct MidConfig {
  int mt, rw, nw, ns;
};

// Up to 64 tokens one M tile of 16 * MT rows covers the tokens, and the
// channels per workgroup (16 * RW) come from a cost model. Each workgroup
// streams its 16 * RW weight rows and loads its 16 * MT token rows, so the
// busiest CU moves rounds(RW) * (16 * RW + 16 * MT) rows, rounds(RW) being
// the workgroups per CU rounded up; the smallest cost wins, ties going to
// fewer channels. For one token group only RW = 1 or 2 compete (64 channels
// measured slower there: 4096 -> 28672 at one token 23.2 against 21.1 us).
// Measured on MI355X over the Llama-3.1-8B and Llama-3-70B projections at M
// in {1, 4, 16, 32, 64}, the model picks the fastest RW everywhere but
// 8192 -> 57344 at M <= 4 (6% behind 16 channels); it reproduces the earlier
// fixed N classes on the 8B shapes and takes 8192 -> 10240 at 32 tokens
// from 24.6 to 21.4 us and at 64 from 31.0 to 26.2. Waves and stages per
// (MT, RW) are the measured best: a fourth stage for K > 8192 at RW = 1,
// 8 waves for 32 tokens at RW = 1 and short K, 2 waves at RW = 4 from 48
// tokens (o at one token: 5.7 against 5.8 us with 8 waves and 4 stages).
//
// From 65 to 128 tokens the kernel runs in M tiles of 64 rows with fixed
// classes of N. Above 128 tokens a workgroup owns 64 channels x 64 tokens,
// with 4 waves (128 KB of LDS, one workgroup per CU) or 2 waves (two per CU,
// each pair taking about 1.5x the time of one 4-wave workgroup, measured on
// the Llama-3.1-8B projections): the one with fewer rounds over the CUs in
// those units (qkv at M = 256, 384 workgroups: 2 waves, 15.7 against
// 20.7 us; at M = 512, 768 workgroups: 4 waves, 30.0 against 31.1 us).
inline MidConfig mid_config(int64_t M, int64_t N, int64_t K, int64_t cus) {
  const bool deep = K > 8192;
  if (M <= kSkinnyMaxM) {
    const int mt = (int)cdiv(M, 16);
    auto cost = [&](int rw) { return cdiv(cdiv(N, 16 * rw), cus) * (16 * rw + 16 * mt); };
    int rw = cost(2) < cost(1) ? 2 : 1;
    if (mt > 1 && cost(4) < cost(rw)) rw = 4;
    switch (mt) {
      case 1:
        if (rw == 2) return {1, 2, 4, 3};
        return deep ? MidConfig{1, 1, 4, 4} : MidConfig{1, 1, 4, 3};
      case 2:
        if (rw == 4) return {2, 4, 4, 3};
        if (rw == 2) return {2, 2, 4, 4};
        return deep ? MidConfig{2, 1, 4, 4} : MidConfig{2, 1, 8, 3};
      case 3:
        if (rw == 4) return {3, 4, 2, 3};
        if (rw == 2) return {3, 2, 4, 3};
        return {3, 1, 4, 3};
      default:
        if (rw == 4) return {4, 4, 2, 2};
        if (rw == 2) return {4, 2, 4, 3};
        return {4, 1, 4, 3};
    }
  }
  if (M <= 128) {
    if (N >= 16384) return {4, 4, 2, 2};
    if (N > 4096) return {4, 4, 4, 2};
    return {4, 2, 4, 3};
  }
  const int64_t groups = cdiv(N, 64) * cdiv(M, 64);
  if (2 * cdiv(groups, cus) <= 3 * cdiv(groups, 2 * cus)) return {4, 4, 4, 2};
  return {4, 4, 2, 2};
}

// Template arguments of the register-staged decode kernel (K % 128 != 0):
// up to 16 * mt tokens and 16 * rw output channels per workgroup, nw waves,
// u 64-byte K chunks in flight per wave, and late scale loads.
struct SkinnyConfig {
  int mt, rw, nw, u;
  bool late;
};

// Shape classes measured on MI355X (Llama-3.1-8B projection shapes). More
// weight rows per wave (RW) reuse each token fragment more often but leave
// fewer workgroups; they pay off once N is large or M > 16. The scales load
// after the weight stream (late) where holding them through it would cost
// a wave per SIMD.
inline SkinnyConfig skinny_config(int64_t M, int64_t N, int64_t K) {
  const bool wide = N > 8192, mid = N > 4096 && N <= 8192, deep = K > 8192;
  if (M <= 4) {
    if (mid) return {1, 2, 8, 8, false};
    if (wide || deep) return {1, 1, 16, 2, false};
    return {1, 1, 16, 8, false};
  }
  if (M <= 16) {
    if (wide) return {1, 4, 8, 2, false};
    if (mid) return {1, 2, 8, 8, true};
    if (deep) return {1, 1, 8, 4, false};
    return {1, 1, 16, 8, false};
  }
  if (M <= 32) {
    if (wide) return {2, 4, 4, 2, true};
    if (mid) return {2, 2, 8, 4, false};
    return {2, 1, 16, 4, false};
  }
  if (M <= 48) {
    if (wide) return {3, 4, 4, 2, false};
    if (mid) return {3, 2, 8, 2, false};
    return {3, 1, 16, 2, false};
  }
  if (wide) return {4, 4, 4, 2, true};
  if (mid) return {4, 2, 8, 2, false};
  if (deep) return {4, 1, 16, 2, false};
  return {4, 1, 8, 8, false};
}

// Tile of the full-line prefill kernel, weight rows x tokens (measured on
// MI355X, Llama-3.1-8B projections at M = 3000 and 4096):
// * when 256 x 256 tiles take one round over the CUs and a three-quarter
//   tile still does, the smaller tile: more CUs, less work each (M = 3000,
//   N = 4096: 256 tiles of 256 x 192 tokens against 192 of 256 x 256,
//   54 against 60 us for K = 4096, 163 against 175 us for K = 14336);
// * otherwise 192 weight rows x 256 tokens when that needs fewer quarter-
//   tile units of rounds (qkv: 103 against 118 us at M = 4096), else
//   256 x 256. Per-tile time shrinks when fewer CUs share the memory
//   system, so more rounds of smaller tiles rarely pay (gate_up at M = 3000:
//   7 rounds of 256 x 192 took 377 us against 6 of 256 x 256 in 370).
enum class PrefillTile { k256x256, k256x192, k192x256 };

inline PrefillTile prefill_tile(int64_t M, int64_t N, int64_t cus) {
  auto tiles = [&](int64_t tn, int64_t tm) { return cdiv(N, tn) * cdiv(M, tm); };
  const int64_t t256 = tiles(256, 256), tm192 = tiles(256, 192), tn192 = tiles(192, 256);
  if (t256 <= cus) {
    if (tm192 <= cus && tm192 > t256) return PrefillTile::k256x192;
    if (tn192 <= cus && tn192 > t256) return PrefillTile::k192x256;
    return PrefillTile::k256x256;
  }
  return 3 * cdiv(tn192, cus) < 4 * cdiv(t256, cus) ? PrefillTile::k192x256
                                                     : PrefillTile::k256x256;
}

}  // namespace dispatch
}  // namespace w8a8
