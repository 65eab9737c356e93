// topk.hip — exact top-K of the indexer scores with a lowest-index
// tie-break, one workgroup per query row.
//
// The TensorRT-LLM QSASparseAttentionConfig reference names an exact radix
// top-K as the default selector over the compressed groups
// (enable_heuristic_topk); the pages give no tie rule, and this library
// ranks by (score descending, group index ascending).  Output per row: the
// min(K, G) selected group ids in ascending order, then -1.
//
// Design (gfx950, one workgroup of 256..1,024 threads per row):
//   * Thread t of NT owns elements t, t + NT, t + 2NT, ... so every load of
//     the score row is fully coalesced; the keys stay in registers for the
//     whole kernel (65,536 groups = 262,144 tokens use 512 threads x 128).
//   * Pass 1 bins the finite scores linearly between their min and max
//     (4,096 LDS bins).  The bin function is monotone in the score, so all
//     elements above the bin that holds the K-th element are selected and
//     only that bin's members stay candidates — usually a handful, and the
//     histogram spreads LDS atomics across many bins.
//   * Three exact radix passes over the order-preserving 32-bit keys of the
//     remaining candidates (11 + 11 + 10 bits) find the K-th key T exactly
//     and how many elements equal to T must be taken.
//   * Compaction in index order uses wave ballots: per (element slot,
//     wave) popcounts are scanned once across the block, which gives every
//     element its rank among equal keys and its output position, so the
//     output is ascending without any sort.
#include "qsa_device.h"
#include "qsa_launch.h"

namespace qsa {
namespace {

constexpr int kBins = 4096;
constexpr int kSlots = 1024;  // (element slot, wave) pairs: E * waves <= 1024

// Inclusive prefix sum across the 64 lanes of a wavefront with DPP: four
// row shifts build 16-lane prefix sums, then row broadcasts of lanes 15 and
// 31 carry them into the next rows.  No address registers are needed.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return x;
}

// Exclusive prefix sum over the block of NT threads; tmp holds NT/64 + 1
// words.  Returns this thread's exclusive prefix.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* tmp) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  const uint32_t x = wave_incl_scan(v);
  if (lane == kWave - 1) tmp[wid] = x;
  __syncthreads();
  if (wid == 0) {
    const uint32_t s = lane < NW ? tmp[lane] : 0u;
    const uint32_t inc = wave_incl_scan(s);
    if (lane < NW) tmp[lane] = inc - s;
  }
  __syncthreads();
  const uint32_t r = tmp[wid] + x - v;
  __syncthreads();
  return r;
}

// In-place exclusive scan of cnt[0..kSlots) by NT threads (each owns
// kSlots / NT consecutive entries).
template <int NT>
__device__ __forceinline__ void scan_slots(uint32_t* cnt, uint32_t* tmp) {
  constexpr int C = kSlots / NT;
  const int tid = threadIdx.x;
  uint32_t v[C], local = 0;
#pragma unroll
  for (int c = 0; c < C; ++c) { v[c] = cnt[tid * C + c]; local += v[c]; }
  uint32_t run = block_excl_scan<NT>(local, tmp);
#pragma unroll
  for (int c = 0; c < C; ++c) { cnt[tid * C + c] = run; run += v[c]; }
  __syncthreads();
}

// Given per-bin counts in hist[0..nbins), find the bin b holding the
// need-th largest element: count(bins > b) < need <= count(bins >= b).
// Writes b and need - count(bins > b) to out[0], out[1].
template <int NT>
__device__ __forceinline__ void find_threshold_bin(const uint32_t* hist, int nbins, uint32_t need,
                                                   uint32_t* tmp, int* out) {
  const int per = nbins / NT;  // bins per thread, >= 1
  const int hi = nbins - per * (int)threadIdx.x;  // thread t covers [hi - per, hi)
  uint32_t local = 0;
  for (int i = 0; i < per; ++i) local += hist[hi - 1 - i];
  uint32_t above = block_excl_scan<NT>(local, tmp);
  if (above < need && need <= above + local) {
    for (int i = 0; i < per; ++i) {
      const uint32_t c = hist[hi - 1 - i];
      if (above + c >= need) {
        out[0] = hi - 1 - i;
        out[1] = (int)(need - above);
        break;
      }
      above += c;
    }
  }
  __syncthreads();
}

// Empty register fence: tells the compiler the keys may have changed, so
// per-element predicates are recomputed in each pass instead of being kept
// alive across passes.
template <int E>
__device__ __forceinline__ void fence_keys(uint32_t (&key)[E]) {
#pragma unroll
  for (int e = 0; e < E; ++e) asm volatile("" : "+v"(key[e]));
}

// NT threads, E keys per thread; element e of thread t is group e*NT + t.
template <int NT, int E>
__global__ __launch_bounds__(NT) void topk_kernel(const float* __restrict__ scores, int gstride,
                                                  const int32_t* __restrict__ row_len,
                                                  int first_pos, int max_ctx, int K,
                                                  int32_t* __restrict__ out) {
  constexpr int NW = NT / kWave;
  static_assert(E * NW <= kSlots, "slot table too small");
  __shared__ uint32_t hist[kBins + 1];  // + dummy bin for slots past the row
  __shared__ uint32_t cnt_eq[kSlots];
  __shared__ uint32_t cnt_sel[kSlots];
  __shared__ uint32_t tmp[NW + 1];
  __shared__ float red[2][NW];
  __shared__ int thr[2];

  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wid = tid / kWave;
  const int L = row_len ? row_len[row] : first_pos + row + 1;
  int G = (L >= 0 && L <= max_ctx) ? L / kRatio : 0;
  if (G > gstride) G = gstride;
  int32_t* orow = out + (size_t)row * K;

  if (G <= K) {  // every complete group is kept
    for (int i = tid; i < K; i += NT) orow[i] = (i < G) ? i : -1;
    return;
  }

  // Unconditional loads (clamped to the row) so all are in flight at once;
  // elements at or past G become key 0 (not a candidate).
  const float* srow = scores + (size_t)row * gstride;
  const int g_rel = G - tid;  // element e is a candidate iff e * NT < g_rel
  const int last = gstride - 1 - tid;
  uint32_t key[E];
#pragma unroll
  for (int e = 0; e < E; ++e) key[e] = __float_as_uint(srow[tid + min(e * NT, last)]);
  fence_keys(key);
#pragma unroll
  for (int e = 0; e < E; ++e)
    key[e] = (e * NT < g_rel) ? score_key(__uint_as_float(key[e])) : 0u;

  // ---- min / max of the finite scores
  float mn = INFINITY, mx = -INFINITY;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const float v = key_value(key[e]);
    const bool ok = (key[e] != 0u) && (fabsf(v) < INFINITY);
    mn = fminf(mn, ok ? v : INFINITY);
    mx = fmaxf(mx, ok ? v : -INFINITY);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    mn = fminf(mn, __shfl_xor(mn, o, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
  }
  if (lane == 0) { red[0][wid] = mn; red[1][wid] = mx; }
  for (int i = tid; i <= kBins; i += NT) hist[i] = 0u;
  __syncthreads();
  mn = red[0][0]; mx = red[1][0];
  for (int w = 1; w < NW; ++w) { mn = fminf(mn, red[0][w]); mx = fmaxf(mx, red[1][w]); }
  float scale = 0.0f;
  if (mx > mn) {
    scale = (float)kBins / (mx - mn);
    if (!(scale < INFINITY)) scale = 0.0f;
  }

  // ---- pass 1: value-linear bins (monotone in the score)
  // Branch-free and monotone non-decreasing in the score: -inf -> 0, values
  // at or above mx -> kBins - 1 (a NaN product, only possible when
  // scale == 0, also lands in bin 0 together with every finite value).
  auto bin_of = [&](uint32_t k) -> int {
    const float t = (key_value(k) - mn) * scale;
    return (int)fminf(fmaxf(t, 0.0f), (float)(kBins - 1));
  };
  fence_keys(key);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    // wave-uniform skip of slots past the row; stragglers count in a dummy bin
    if (e * NT + wid * kWave < G) atomicAdd(&hist[key[e] ? bin_of(key[e]) : kBins], 1u);
    __builtin_amdgcn_sched_barrier(0);
  }
  __syncthreads();
  find_threshold_bin<NT>(hist, kBins, (uint32_t)K, tmp, thr);
  const int tb = thr[0];
  uint32_t need = (uint32_t)thr[1];

  // The keys whose bin is tb form one contiguous key range [lo, hi]
  // (the bin function is monotone in the key between key(-inf) and
  // key(+inf)); one thread finds its ends by bisection, so candidates are
  // tested by two compares instead of re-binning every element.
  if (tid == 0) {
    const uint32_t kneg = score_key(-INFINITY), kpos = score_key(INFINITY);
    uint32_t a = kneg, b = kpos;  // smallest key with bin >= tb
    while (a < b) {
      const uint32_t m = a + (b - a) / 2;
      if (bin_of(m) >= tb) b = m; else a = m + 1;
    }
    uint32_t c = kneg, d = kpos;  // largest key with bin <= tb
    while (c < d) {
      const uint32_t m = c + (d - c + 1) / 2;
      if (bin_of(m) <= tb) c = m; else d = m - 1;
    }
    thr[0] = (int)a;
    thr[1] = (int)c;
  }
  __syncthreads();
  uint32_t lo = (uint32_t)thr[0], hi = (uint32_t)thr[1];

  // ---- passes 2-4: exact radix over the candidates' keys; each pass
  // narrows [lo, hi] to the keys that share the chosen digit prefix
  const int shifts[3] = {21, 10, 0};
  const int widths[3] = {11, 11, 10};
#pragma unroll
  for (int p = 0; p < 3; ++p) {
    const int sh = shifts[p];
    const uint32_t dmask = (1u << widths[p]) - 1u;
    const int nb = 1 << widths[p];
    __syncthreads();
    for (int i = tid; i < nb; i += NT) hist[i] = 0u;
    __syncthreads();
    fence_keys(key);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (key[e] >= lo && key[e] <= hi) atomicAdd(&hist[(key[e] >> sh) & dmask], 1u);
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
    find_threshold_bin<NT>(hist, nb, need, tmp, thr);
    const uint32_t d = (uint32_t)thr[0];
    need = (uint32_t)thr[1];
    const uint32_t top = ~((dmask << sh) | ((1u << sh) - 1u));  // bits above the digit
    const uint32_t base = (lo & top) | (d << sh);
    lo = max(lo, base);
    hi = min(hi, base | ((1u << sh) - 1u));
  }
  const uint32_t prefix = lo;
  const uint32_t T = prefix;  // the K-th largest key; take `need` of its copies

  // ---- compaction in index order.  Element e of thread t has index
  // e * NT + t, so index order is (slot e, wave, lane): per (e, wave) ballot
  // popcounts scanned across the block give each element its rank among
  // the keys equal to T and then its output position.  Ballots are
  // recomputed rather than stored.
  const uint64_t lt = (1ull << lane) - 1ull;
  fence_keys(key);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint64_t eqb = __ballot(key[e] == T);
    if (lane == 0) cnt_eq[e * NW + wid] = (uint32_t)__popcll(eqb);
  }
  for (int i = E * NW + tid; i < kSlots; i += NT) cnt_eq[i] = 0u;
  __syncthreads();
  scan_slots<NT>(cnt_eq, tmp);
  // Per-slot bases are wave-uniform: lane l holds the base of slot l (and
  // l + 64), and each slot reads it back with v_readlane into a scalar.
  constexpr int NV = (E + kWave - 1) / kWave;
  uint32_t eq_base[NV], sel_base[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int e = v * kWave + lane;
    eq_base[v] = e < E ? cnt_eq[e * NW + wid] : 0u;
  }
  auto taken = [&](int e) -> bool {
    const uint64_t eqb = __ballot(key[e] == T);
    const uint32_t base = (uint32_t)__builtin_amdgcn_readlane((int)eq_base[e / kWave], e % kWave);
    if (key[e] == T) return base + (uint32_t)__popcll(eqb & lt) < need;
    return key[e] > T;
  };
  fence_keys(key);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint64_t selb = __ballot(taken(e));
    if (lane == 0) cnt_sel[e * NW + wid] = (uint32_t)__popcll(selb);
  }
  for (int i = E * NW + tid; i < kSlots; i += NT) cnt_sel[i] = 0u;
  __syncthreads();
  scan_slots<NT>(cnt_sel, tmp);
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int e = v * kWave + lane;
    sel_base[v] = e < E ? cnt_sel[e * NW + wid] : 0u;
  }
  fence_keys(key);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool t = taken(e);
    const uint64_t selb = __ballot(t);
    if (t) {
      const uint32_t base = (uint32_t)__builtin_amdgcn_readlane((int)sel_base[e / kWave], e % kWave);
      const uint32_t pos = base + (uint32_t)__popcll(selb & lt);
      if (pos < (uint32_t)K) orow[pos] = e * NT + tid;
    }
  }
}

}  // namespace

hipError_t launch_topk(const float* scores, int gstride, int n_rows, const int32_t* row_len,
                       int first_pos, int max_ctx, int K, int32_t* out, hipStream_t stream) {
  if (n_rows <= 0) return hipSuccess;
  dim3 grid(n_rows);
#define QSA_TOPK_CASE(NT, EV)                                                                   \
  if (gstride <= (NT) * (EV)) {                                                                 \
    hipLaunchKernelGGL((topk_kernel<NT, EV>), grid, dim3(NT), 0, stream, scores, gstride,      \
                       row_len, first_pos, max_ctx, K, out);                                    \
    return hipGetLastError();                                                                   \
  }
  QSA_TOPK_CASE(256, 4)
  QSA_TOPK_CASE(256, 16)
  QSA_TOPK_CASE(512, 16)
  QSA_TOPK_CASE(1024, 16)
  QSA_TOPK_CASE(1024, 32)
  QSA_TOPK_CASE(1024, 64)
#undef QSA_TOPK_CASE
  return hipErrorInvalidValue;
}

}  // namespace qsa
