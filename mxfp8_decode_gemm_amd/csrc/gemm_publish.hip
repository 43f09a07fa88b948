// Host side of the publishing GEMM (the kernel is in gemm_kernel.h): the
// weight packing kernels, the variant table lookup, the tile chooser and the
// launcher.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <tuple>

#include "gemm_kernel.h"

namespace mxg {
namespace {

// Packs row-major W [n, k] and its scales [n, k/32] into the tile layout the
// GEMM streams: row block rb (16 rows, zero rows past n), K block kb (128):
//   w_packed  + (rb*K/128 + kb)*2048 + h*1024 + 16*l : 16 bytes of row
//             rb*16 + l%16, K = kb*128 + 64*h + 16*(l/16) .. +16
//   ws_packed + ((rb*K/128 + kb)*16 + r)*4            : the 4 scale bytes of
//             row rb*16 + r for that K block (byte 127 past n)
// One thread per 16-byte chunk; every index is checked against the sizes.
__global__ void pack_weight_kernel(const uint8_t* w, const uint8_t* ws, int n, int k,
                                   uint8_t* wp, uint8_t* wsp) {
  const int kbt = k >> 7;
  const int rbn = (n + 15) >> 4;
  const size_t chunks = (size_t)rbn * kbt * 128;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t c = (size_t)blockIdx.x * blockDim.x + threadIdx.x; c < chunks; c += stride) {
    const size_t t = c >> 7;
    const int within = (int)(c & 127);
    const int h = within >> 6, l = within & 63;
    const int rb = (int)(t / kbt), kb = (int)(t - (size_t)rb * kbt);
    const int row = rb * 16 + (l & 15);
    uint4 v = {0u, 0u, 0u, 0u};
    if (row < n)
      v = *reinterpret_cast<const uint4*>(w + (size_t)row * k + kb * 128 + 64 * h + 16 * (l >> 4));
    reinterpret_cast<uint4*>(wp)[c] = v;
    if (within < 16) {
      const int r = within;
      const int srow = rb * 16 + r;
      uint32_t s = 0x7F7F7F7Fu;
      if (srow < n)
        s = *reinterpret_cast<const uint32_t*>(ws + (size_t)srow * (k >> 5) + kb * 4);
      reinterpret_cast<uint32_t*>(wsp)[t * 16 + r] = s;
    }
  }
}

// The word per 16-row block that follows the packed scale tiles: over the
// block's (row, 32-wide K block) pairs that hold a nonzero code, the
// smallest scale byte in bits 0-7 and the largest in bits 8-15 (0xFF and 0
// when there is none). The GEMM checks them against the range its main loop
// keeps exact; a block of zero codes contributes zeros at any scale. One wave
// per row block, after pack_weight_kernel on the same stream. In a packed
// tile, lane l's 16-byte pieces at 16 l and 1024 + 16 l hold row l % 16 and K
// 16 (l / 16) .. +16 and 64 + 16 (l / 16) .. +16, so lanes l and l ^ 16 hold
// the two halves of the 32-wide blocks l / 32 and 2 + l / 32 of row l % 16.
__global__ void scale_summary_kernel(const uint8_t* wp, const uint8_t* wsp, int rbn, int kbt,
                                     uint32_t* summary) {
  const int rb = blockIdx.x * (blockDim.x >> 6) + (int)(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (rb >= rbn) return;  // whole waves
  uint32_t lo = 255u, hi = 0u;
  for (int kb = 0; kb < kbt; ++kb) {
    const size_t t = (size_t)rb * kbt + kb;
    const uint4 p0 = *reinterpret_cast<const uint4*>(wp + t * 2048 + 16 * lane);
    const uint4 p1 = *reinterpret_cast<const uint4*>(wp + t * 2048 + 1024 + 16 * lane);
    uint32_t nz0 = ((p0.x | p0.y | p0.z | p0.w) & 0x7F7F7F7Fu) != 0 ? 1u : 0u;
    uint32_t nz1 = ((p1.x | p1.y | p1.z | p1.w) & 0x7F7F7F7Fu) != 0 ? 1u : 0u;
    nz0 |= (uint32_t)__shfl_xor((int)nz0, 16, 64);
    nz1 |= (uint32_t)__shfl_xor((int)nz1, 16, 64);
    const uint32_t sw = reinterpret_cast<const uint32_t*>(wsp)[t * 16 + (lane & 15)];
    const uint32_t s0 = (sw >> (8 * (lane >> 5))) & 0xFFu;
    const uint32_t s1 = (sw >> (8 * (2 + (lane >> 5)))) & 0xFFu;
    if (nz0) {
      lo = s0 < lo ? s0 : lo;
      hi = s0 > hi ? s0 : hi;
    }
    if (nz1) {
      lo = s1 < lo ? s1 : lo;
      hi = s1 > hi ? s1 : hi;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t l2 = (uint32_t)__shfl_xor((int)lo, o, 64);
    const uint32_t h2 = (uint32_t)__shfl_xor((int)hi, o, 64);
    lo = l2 < lo ? l2 : lo;
    hi = h2 > hi ? h2 : hi;
  }
  if (lane == 0) summary[rb] = lo | (hi << 8);
}

const void* variant_fn(const Variant& v, bool bf16_x, bool x16) {
  return x16 ? (bf16_x ? v.fn16_q : v.fn16) : (bf16_x ? v.fn_q : v.fn);
}

const Variant* find_variant(const TileCfg& c, int split_k) {
  static const Variant* (*const kParts[kVariantParts])(size_t*) = {gemm_variants_0, gemm_variants_1, gemm_variants_2, gemm_variants_3, gemm_variants_4, gemm_variants_5};
  for (auto part : kParts) {
    size_t count = 0;
    const Variant* vs = part(&count);
    for (size_t i = 0; i < count; ++i) {
      const Variant& v = vs[i];
      if (v.cfg.rb == c.rb && v.cfg.wn == c.wn && v.cfg.wk == c.wk && v.cfg.depth == c.depth &&
        v.cfg.xr == c.xr &&
        v.split_k == split_k)
        return &v;
    }
  }
  return nullptr;
}

}  // namespace

size_t gemm_lds_bytes(const TileCfg& c, int m, int k_slice) {
  const size_t xbytes =
      c.x16 ? 2 * (size_t)m * k_slice : (size_t)m * k_slice + (size_t)m * (k_slice / 32);
  const size_t red = (size_t)c.wk * m * tile_rows(c) * sizeof(float);
  return kHeaderBytes + std::max(xbytes, red);
}

bool tile_available(const TileCfg& c) { return find_variant(c, 1) != nullptr; }

static bool choose_tile_uncached(int m, int n, int k, int split_k, const char* tile,
                                 TileCfg* out);

// The default choice depends only on the sizes and the device: remembered
// per key (a memo of device queries, not state that changes a result). A
// forced tile is not remembered.
bool choose_tile(int m, int n, int k, int split_k, const char* tile, TileCfg* out) {
  if (tile) return choose_tile_uncached(m, n, k, split_k, tile, out);
  static std::mutex mu;
  static std::map<std::tuple<int, int, int, int, int>, std::pair<bool, TileCfg>> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  const auto key = std::make_tuple(dev, m, n, k, split_k);
  {
    std::lock_guard<std::mutex> g(mu);
    auto it = cache.find(key);
    if (it != cache.end()) {
      *out = it->second.second;
      return it->second.first;
    }
  }
  TileCfg c{};
  const bool ok = choose_tile_uncached(m, n, k, split_k, nullptr, &c);
  std::lock_guard<std::mutex> g(mu);
  cache[key] = std::make_pair(ok, c);
  *out = c;
  return ok;
}

static bool choose_tile_uncached(int m, int n, int k, int split_k, const char* tile,
                                 TileCfg* out) {
  const int ks = k / split_k;
  auto fits = [&](const TileCfg& c) {
    const Variant* v = find_variant(c, split_k);
    if (!v || (c.x16 && !v->fn16) || gemm_lds_bytes(c, m, ks) > 160 * 1024) return false;
    if (split_k == 1) return true;
    // The workgroups of one tile wait for each other: the grid must be
    // resident all at once.
    const long tiles = (n + tile_rows(c) - 1) / tile_rows(c);
    const long resident = gemm_resident_blocks(c, split_k, gemm_lds_bytes(c, m, ks));
    return resident > 0 && tiles * split_k <= resident && tiles * split_k <= MXG_WS_MAX_GROUPS;
  };
  int cus = 256;
  {
    int dev = 0;
    if (hipGetDevice(&dev) == hipSuccess)
      (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (cus < 1) cus = 1;
  }
  // x staged as BF16 when the variant has it, it fits (with split-K: and the
  // grid stays resident), and each CU runs at most one workgroup: measured
  // 0.3-0.6 us faster on N=7168/K=2048/m=4, N=2048/K=8192/m=8/S=4 and
  // N=256/K=512/m=1 and on BF16 x, neutral on N=7168/K=8192/m=8/S=4, and
  // 3-4 us slower on N=4096/K=16384/S=8, where two workgroups share a CU.
  // The tile spec "fp8" keeps the FP8 stage.
  const bool keep_fp8 = tile && std::strcmp(tile, "fp8") == 0;
  auto upgrade_x16 = [&](TileCfg& c) {
    if (keep_fp8) return;
    const long grid = (long)((n + tile_rows(c) - 1) / tile_rows(c)) * split_k;
    if (grid > cus) return;
    TileCfg c2 = c;
    c2.x16 = 1;
    if (fits(c2)) c = c2;
  };
  if (tile && !keep_fp8) {
    // Forced variant (mxgemm_tile): exactly "rb,wn,wk,depth[,xr[,x16]]", x16
    // chosen as usual when not given, or no launch at all.
    TileCfg c{};
    const int got =
        std::sscanf(tile, "%d,%d,%d,%d,%d,%d", &c.rb, &c.wn, &c.wk, &c.depth, &c.xr, &c.x16);
    if (got == 4) c.xr = 1;
    if (got < 6) c.x16 = 0;
    if (got < 4 || (c.x16 != 0 && c.x16 != 1) || !fits(c)) return false;
    if (got < 6) upgrade_x16(c);
    *out = c;
    return true;
  }
  // Cost of a candidate: the W bytes one CU streams, plus a fixed cost per
  // workgroup (x staging, exchange, publish), times the workgroups each CU
  // runs. Lists are in preference order for ties; shallow rings (3 K blocks
  // per wave) first, since they keep the workgroups' progress even when the
  // whole chip's loads are queued at once. Fitted to sweeps of every variant
  // on N=7168/K=8192/m=8/S=4, N=7168/K=2048/m=4, N=4096/K=16384 (m 1..8,
  // S 1/4/8), N=7168/K=4096/m=1/S=4 and N=2048/K=8192/m=8/S=4.
  // After the B operand stopped being converted in every wave, deeper rings
  // paid on the 112- and 32-row tiles (depth 5: N=7168/K=8192/m=8/S=4 14.3 ->
  // 13.95 us, N=7168/K=2048/m=4 6.5 -> 6.1 us, N=2048/K=8192/m=8/S=4 8.5 ->
  // 8.2 us) and not on the 64-row one.
  static const TileCfg kSplit[] = {{1, 7, 1, 5}, {1, 4, 1, 3}, {1, 2, 2, 5}, {1, 7, 1, 3},
                                   {1, 2, 2, 8}, {1, 7, 1, 4}, {1, 4, 1, 8}, {1, 4, 2, 8},
                                   {2, 1, 4, 4}, {1, 1, 4, 4}};
  // Without split-K the 16- and 8-wave 16-row tiles tie in the cost below;
  // measured on N=4096/K=16384, the 8-wave one is faster up to 4 tokens
  // (m=1: 14.9 against 16.6 us, m=4: 16.1 against 16.8 us) and the 16-wave
  // one at 8 (17.4 against 18.2 us).
  static const TileCfg kNoSplit[] = {{1, 1, 16, 4}, {1, 1, 8, 4}, {1, 2, 2, 5}, {1, 2, 2, 8},
                                     {1, 4, 1, 3}, {1, 1, 4, 4}, {2, 1, 4, 4}};
  static const TileCfg kNoSplitFew[] = {{1, 1, 8, 4}, {1, 1, 16, 4}, {1, 2, 2, 5}, {1, 2, 2, 8},
                                        {1, 4, 1, 3}, {1, 1, 4, 4}, {2, 1, 4, 4}};
  const TileCfg* list = split_k > 1 ? kSplit : (m <= 4 ? kNoSplitFew : kNoSplit);
  const size_t count = split_k > 1 ? sizeof(kSplit) / sizeof(kSplit[0])
                                   : sizeof(kNoSplit) / sizeof(kNoSplit[0]);
  constexpr double kGroupCost = 32768.0;  // bytes-equivalent fixed cost per workgroup
  bool found = false;
  double best = 0.0;
  for (size_t i = 0; i < count; ++i) {
    const TileCfg& c = list[i];
    if (c.wk > ks / 128 || !fits(c)) continue;  // every wave along K gets a K block
    const long grid = (long)((n + tile_rows(c) - 1) / tile_rows(c)) * split_k;
    const long per_cu = (grid + cus - 1) / cus;
    const double cost = (double)per_cu * ((double)tile_rows(c) * ks + kGroupCost);
    if (!found || cost < best) {
      best = cost;
      *out = c;
      found = true;
    }
  }
  // A slice of x that needs more than one staging round of 4 chunks per
  // thread: the variant with an 8-chunk first round, when built and resident
  // (N=4096/K=16384/m=8: S=4 17.5 -> 16.8 us; S=1 on the 16-wave tile
  // 18.6 -> 18.0 us).
  if (found) {
    const long chunks = (long)m * (ks / 16);
    TileCfg c2 = *out;
    c2.xr = 2;
    if (chunks > 4L * 64 * out->wn * out->wk && fits(c2)) *out = c2;
    upgrade_x16(*out);
  }
  return found;
}

long gemm_resident_blocks(const TileCfg& c, int split_k, size_t lds_bytes) {
  static std::mutex mu;
  static std::map<std::tuple<int, int, int, int, int, size_t>, long> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  const auto key = std::make_tuple(dev, c.rb, c.wn,
                                   c.wk * 100 + c.depth + 10000 * c.xr + 100000 * c.x16, split_k,
                                   lds_bytes);
  {
    std::lock_guard<std::mutex> g(mu);
    auto it = cache.find(key);
    if (it != cache.end()) return it->second;
  }
  const Variant* v = find_variant(c, split_k);
  if (!v) return -1;
  // Both activation forms of the variant: a shape gets one tile either way.
  int per_cu = 1 << 30, cus = 0;
  for (const void* fn : {variant_fn(*v, false, c.x16), variant_fn(*v, true, c.x16)}) {
    int n = 0;
    if (!fn) return -1;
    if (lds_bytes > 64 * 1024 &&
        hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes) !=
            hipSuccess)
      return -1;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, tile_threads(c, split_k),
                                                     lds_bytes) != hipSuccess)
      return -1;
    per_cu = n < per_cu ? n : per_cu;
  }
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return -1;
  const long r = (long)per_cu * cus;
  std::lock_guard<std::mutex> g(mu);
  cache[key] = r;
  return r;
}

hipError_t launch_pack_weight(const uint8_t* w, const uint8_t* ws, int n, int k, uint8_t* wp,
                              uint8_t* wsp, hipStream_t s) {
  const size_t chunks = (size_t)((n + 15) / 16) * (k / 128) * 128;
  const size_t blocks = std::min<size_t>((chunks + 255) / 256, 65536);
  hipLaunchKernelGGL(pack_weight_kernel, dim3((unsigned)blocks), dim3(256), 0, s, w, ws, n, k,
                     wp, wsp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int rbn = (n + 15) / 16, kbt = k / 128;
  hipLaunchKernelGGL(scale_summary_kernel, dim3((unsigned)((rbn + 3) / 4)), dim3(256), 0, s, wp,
                     wsp, rbn, kbt, reinterpret_cast<uint32_t*>(wsp + (size_t)rbn * kbt * 64));
  return hipGetLastError();
}

hipError_t launch_gemm_publish(const GemmArgs& a, const TileCfg& c, hipStream_t s,
                               hipEvent_t ev_start, hipEvent_t ev_stop) {
  const Variant* v = find_variant(c, a.split_k);
  if (!v) return hipErrorInvalidValue;
  const int tiles = (a.n + tile_rows(c) - 1) / tile_rows(c);
  const dim3 grid(tiles * a.split_k), block(tile_threads(c, a.split_k));
  const size_t lds = gemm_lds_bytes(c, a.m, a.k / a.split_k);
  GemmArgs args = a;
  args.xcd_groups = a.split_k > 1 && tiles % 8 == 0 ? 1 : 0;
  const void* fn = variant_fn(*v, a.xb != nullptr, c.x16);
  if (!fn) return hipErrorInvalidValue;
  if (lds > 64 * 1024) {
    const hipError_t e =
        hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  void* kargs[] = {&args};
  if (ev_start || ev_stop)
    return hipExtLaunchKernel(fn, grid, block, kargs, lds, s, ev_start, ev_stop, 0);
  return hipLaunchKernel(fn, grid, block, kargs, lds, s);
}

}  // namespace mxg
