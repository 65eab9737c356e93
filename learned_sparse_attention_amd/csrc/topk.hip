// topk.hip — exact top-K of the indexer scores with a lowest-index
// tie-break.
//
// The TensorRT-LLM QSASparseAttentionConfig reference names an exact radix
// top-K as the default selector over the compressed groups
// (enable_heuristic_topk); the pages give no tie rule, and this library
// ranks by (score descending, group index ascending).  Output per row: the
// min(K, G) selected group ids in ascending order, then -1.
//
// Four paths, by the length of the score rows:
//   up to 2,048 groups (short decode contexts, early prefill queries):
//            one wavefront per row.  Lane l holds 32 consecutive groups;
//            the K-th key comes from radix passes over a wave-owned
//            histogram, the selection from bit masks and wave scans.
//   up to 8,192 groups (a prefill chunk's thousands of rows): one
//            256-thread workgroup per row (row kernel).  The row is pruned
//            with a sampled guess (below) inside the workgroup and only the
//            candidates are ranked.
//   up to 16,384 groups (a few decode rows): the row kernel with 512
//            threads.
//   longer (decode at long context: up to 65,536 groups per row, a handful
//            of rows): spread over many compute units in two launches.
//   extract  one workgroup per 4,096-group slice.  Every slice of a row
//            derives the same pruning threshold ("guess") from 512 evenly
//            spaced sample scores of the row: an exact radix select of the
//            r-th largest sample, with r = the sample rank of K plus four
//            standard deviations of its sampling error, so the guess lies
//            below the K-th largest score with overwhelming probability.
//            The slice then writes every score >= guess (typically ~6.6% at
//            K/G = 1/32) with its index to its own region of the workspace,
//            and records its count, its largest key and the guess.
//   finish   one workgroup per row gathers the candidates (~4K), finds the
//            K-th key T exactly with radix passes of up to 12 bits over the
//            key offsets from the guess, marks key > T and key == T in LDS
//            bitmaps, and emits ascending indices, copies of T in index
//            order, through a block scan of bitmap popcounts.
// Whenever a guess misses (a slice or a wave's candidate region overflows,
// or fewer than K candidates survive), the row is ranked exactly from all of
// its scores instead, so the result never depends on the sample.
#include "qsa_device.h"
#include "qsa_launch.h"

namespace qsa {
namespace {

constexpr int kSlice = 4096;       // groups per extract workgroup
constexpr int kSliceCap = 1024;    // candidate slots per slice
constexpr int kSample = 512;       // sample scores per row
constexpr int kDirect = 16384;     // rows up to this length skip extraction
constexpr int kMaxGroups = 65536;  // 262,144 tokens / 4
constexpr int kMaxSlices = kMaxGroups / kSlice;
constexpr int kFinishThreads = 1024;
constexpr int kWaveRow = 2048;     // rows up to this length: one wavefront per row
constexpr int kShort = 8192;       // rows up to this length: kShortThreads per row
constexpr int kShortThreads = 256;
constexpr int kRowCap = 4096;      // candidate slots of a short row
constexpr int kExtractThreads = 256;
constexpr int kBins = 4096;        // fallback value-linear bins
constexpr int kInfo = 4;           // per (row, slice): count, largest key, guess key, unused

// Inclusive prefix sum across the 64 lanes of a wavefront with DPP: four
// row shifts build 16-lane prefix sums, then row broadcasts of lanes 15 and
// 31 carry them into the next rows.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return x;
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, o, kWave));
  return v;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, kWave));
  return v;
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

// Wave-level search of a 256-bin histogram for the bin holding the
// need-th largest element: count(bins > b) < need <= count(bins >= b).
// Lane l owns bins [252 - 4l, 256 - 4l).  Every lane gets b and
// need - count(bins > b).
__device__ __forceinline__ void wave_find256(const uint32_t* hist, uint32_t need, uint32_t* bin,
                                             uint32_t* rem) {
  const int lane = threadIdx.x & (kWave - 1);
  const int lo = 252 - 4 * lane;
  const uint4 v = *reinterpret_cast<const uint4*>(hist + lo);
  const uint32_t local = (v.x + v.y) + (v.z + v.w);
  const uint32_t incl = wave_incl_scan(local);
  const bool mine = incl - local < need && need <= incl;
  uint32_t r = need - (incl - local);
  uint32_t b = lo;
  if (r <= v.w) b = lo + 3;
  else if ((r -= v.w) <= v.z) b = lo + 2;
  else if ((r -= v.z) <= v.y) b = lo + 1;
  else r -= v.y;
  const uint64_t m = __ballot(mine);
  const int src = m ? __ffsll((unsigned long long)m) - 1 : 0;
  *bin = (uint32_t)__shfl((int)b, src, kWave);
  *rem = (uint32_t)__shfl((int)r, src, kWave);
}

// Block-level 256-bin search (wave 0 searches; result through sh).
__device__ __forceinline__ void block_find256(const uint32_t* hist, uint32_t need, int* sh,
                                              uint32_t* bin, uint32_t* rem) {
  if (threadIdx.x < kWave) {
    uint32_t b, r;
    wave_find256(hist, need, &b, &r);
    if (threadIdx.x == 0) { sh[0] = (int)b; sh[1] = (int)r; }
  }
  __syncthreads();
  *bin = (uint32_t)sh[0];
  *rem = (uint32_t)sh[1];
  __syncthreads();
}

// r-th largest of M keys per lane of one wave (64 M keys; key 0 = empty
// slot never counts), exact: four 8-bit radix passes with an LDS histogram
// owned by this wave alone (LDS operations of one wave execute in order, so
// no barrier is needed).
template <int M>
__device__ uint32_t wave_select_rth(const uint32_t (&k)[M], uint32_t r, uint32_t* hist) {
  const int lane = threadIdx.x & (kWave - 1);
  uint32_t prefix = 0, pmask = 0;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int s = 24 - 8 * p;
    *reinterpret_cast<uint4*>(hist + 4 * lane) = make_uint4(0u, 0u, 0u, 0u);
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < M; ++i)
      if (k[i] && (k[i] & pmask) == prefix) atomicAdd(&hist[(k[i] >> s) & 255u], 1u);
    __builtin_amdgcn_wave_barrier();
    uint32_t b;
    wave_find256(hist, r, &b, &r);
    __builtin_amdgcn_wave_barrier();
    prefix |= b << s;
    pmask |= 255u << s;
  }
  return prefix;
}

// r-th largest of the M keys per lane of one wave (0 = empty slot), like
// wave_select_rth, but with radix passes of 8 bits over the offsets
// key - kmin within the span of the present keys: a row's scores share a
// few binary exponents, so the top digit of the raw keys would send almost
// every key to two or three bins and serialise the LDS atomics.
template <int M>
__device__ uint32_t wave_select_span(const uint32_t (&k)[M], uint32_t r, uint32_t* hist) {
  const int lane = threadIdx.x & (kWave - 1);
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int i = 0; i < M; ++i)
    if (k[i]) { kmin = min(kmin, k[i]); kmax = max(kmax, k[i]); }
  kmin = wave_min_u32(kmin);
  kmax = wave_max_u32(kmax);
  const uint32_t span = kmax >= kmin ? kmax - kmin : 0u;
  int nbits = span ? 32 - __clz(span) : 0;
  uint32_t prefix = 0, pmask = 0;
  while (nbits > 0) {
    const int s = nbits > 8 ? nbits - 8 : 0;
    const uint32_t dmask = (1u << (nbits - s)) - 1u;
    *reinterpret_cast<uint4*>(hist + 4 * lane) = make_uint4(0u, 0u, 0u, 0u);
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < M; ++i) {
      const uint32_t off = k[i] - kmin;
      if (k[i] && (off & pmask) == prefix) atomicAdd(&hist[(off >> s) & dmask], 1u);
    }
    __builtin_amdgcn_wave_barrier();
    uint32_t b;
    wave_find256(hist, r, &b, &r);
    __builtin_amdgcn_wave_barrier();
    prefix |= b << s;
    pmask |= dmask << s;
    nbits = s;
  }
  return kmin + prefix;
}

// Exact threshold among the M keys per thread of a whole short row (0 =
// empty slot): the need-th largest key T and how many copies of T are
// taken.  Scores of a row crowd into a few binary exponents, so radix
// digits of the keys would pile into a handful of histogram bins; the first
// pass instead sorts the keys into 256 bins linear in the score between the
// row's finite minimum and maximum (a monotone map of the key: -inf and
// below to bin 0, +inf and above to bin 255), then radix passes over the
// key offsets rank the keys of the bin that holds the need-th one.
template <int NT, int M>
__device__ uint32_t row_threshold(const uint32_t (&key)[M], uint32_t need, uint32_t* hist,
                                  float* red, int* sh, uint32_t* take_eq) {
  static_assert(M <= 32, "one bit per key in a mask");
  constexpr int NW = NT / kWave;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const uint32_t kneg = score_key(-INFINITY), kpos = score_key(INFINITY);
  float mn = INFINITY, mx = -INFINITY;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    if (key[m] > kneg && key[m] < kpos) {
      const float v = key_value(key[m]);
      mn = fminf(mn, v);
      mx = fmaxf(mx, v);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    mn = fminf(mn, __shfl_xor(mn, o, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
  }
  if (lane == 0) { red[wid] = mn; red[NW + wid] = mx; }
  for (int i = tid; i < 256; i += NT) hist[i] = 0u;
  if (tid == 0) { sh[2] = (int)0xFFFFFFFFu; sh[3] = 0; }
  __syncthreads();
  mn = red[0]; mx = red[NW];
  for (int w = 1; w < NW; ++w) { mn = fminf(mn, red[w]); mx = fmaxf(mx, red[NW + w]); }
  float scale = 0.0f;
  if (mx > mn) {
    scale = 256.0f / (mx - mn);
    if (!(scale < INFINITY)) scale = 0.0f;
  }
  auto bin_of = [&](uint32_t k) -> uint32_t {
    if (k <= kneg) return 0u;
    if (k >= kpos) return 255u;
    const float t = (key_value(k) - mn) * scale;
    return (uint32_t)fminf(fmaxf(t, 0.0f), 255.0f);
  };
#pragma unroll
  for (int m = 0; m < M; ++m)
    if (key[m]) atomicAdd(&hist[bin_of(key[m])], 1u);
  __syncthreads();
  uint32_t tb;
  block_find256(hist, need, sh, &tb, &need);
  // key range of the chosen bin, and which of this thread's keys lie in it
  uint32_t in_bin = 0u, lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    if (key[m] && bin_of(key[m]) == tb) {
      in_bin |= 1u << m;
      lo = min(lo, key[m]);
      hi = max(hi, key[m]);
    }
  }
  lo = wave_min_u32(lo);
  hi = wave_max_u32(hi);
  if (lane == 0 && lo <= hi) {
    atomicMin(reinterpret_cast<uint32_t*>(&sh[2]), lo);
    atomicMax(reinterpret_cast<uint32_t*>(&sh[3]), hi);
  }
  __syncthreads();
  lo = (uint32_t)sh[2];
  hi = (uint32_t)sh[3];
  const uint32_t span = hi - lo;
  int nbits = span ? 32 - __clz(span) : 0;
  uint32_t prefix = 0, pmask = 0;  // over offsets key - lo
  while (nbits > 0) {
    const int sft = nbits > 8 ? nbits - 8 : 0;
    const uint32_t dmask = (1u << (nbits - sft)) - 1u;
    for (int i = tid; i < 256; i += NT) hist[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const uint32_t off = key[m] - lo;
      if (((in_bin >> m) & 1u) && (off & pmask) == prefix)
        atomicAdd(&hist[(off >> sft) & dmask], 1u);
    }
    __syncthreads();
    uint32_t d;
    block_find256(hist, need, sh, &d, &need);
    prefix |= d << sft;
    pmask |= dmask << sft;
    nbits = sft;
  }
  *take_eq = need;
  return lo + prefix;
}

// Exact threshold over all G scores of a row, streamed from memory in
// every pass (the rare path taken when the pruning guess misses): the
// need-th largest key T and how many copies of T are taken.  Keys are
// ranked by value-linear bins first (4,096 bins between min and max of the
// finite scores; monotone in the score), then by three radix digits of the
// keys inside the bin that holds the need-th one.
template <int NT>
__device__ uint32_t exact_threshold_stream(const float* srow, int G, uint32_t need, uint32_t* hist,
                                           float* red, int* sh, uint32_t* take_eq) {
  constexpr int NW = NT / kWave;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  float mn = INFINITY, mx = -INFINITY;
  for (int i = tid; i < G; i += NT) {
    const float v = srow[i];
    const bool ok = fabsf(v) < INFINITY;
    mn = fminf(mn, ok ? v : INFINITY);
    mx = fmaxf(mx, ok ? v : -INFINITY);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    mn = fminf(mn, __shfl_xor(mn, o, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
  }
  if (lane == 0) { red[wid] = mn; red[NW + wid] = mx; }
  for (int i = tid; i < kBins; i += NT) hist[i] = 0u;
  __syncthreads();
  mn = red[0]; mx = red[NW];
  for (int w = 1; w < NW; ++w) { mn = fminf(mn, red[w]); mx = fmaxf(mx, red[NW + w]); }
  __syncthreads();
  float scale = 0.0f;
  if (mx > mn) {
    scale = (float)kBins / (mx - mn);
    if (!(scale < INFINITY)) scale = 0.0f;
  }
  // Branch-free and monotone non-decreasing in the score: -inf -> 0, values
  // at or above mx -> kBins - 1 (a NaN product, only possible when
  // scale == 0, lands in bin 0 together with every finite value).
  auto bin_of = [&](uint32_t k) -> int {
    const float t = (key_value(k) - mn) * scale;
    return (int)fminf(fmaxf(t, 0.0f), (float)(kBins - 1));
  };
  for (int i = tid; i < G; i += NT) atomicAdd(&hist[bin_of(score_key(srow[i]))], 1u);
  __syncthreads();
  // bin holding the need-th largest: 16 coarse groups of 256 bins, then fine
  if (tid < kWave) {
    uint32_t above = 0;
    int b = 0;
    for (int grp = 15; grp >= 0; --grp) {
      uint32_t c = 0;
      for (int i = tid; i < 256; i += kWave) c += hist[grp * 256 + i];
      c = wave_incl_scan(c);
      c = (uint32_t)__shfl((int)c, kWave - 1, kWave);
      if (above + c >= need) {
        uint32_t bb, rr;
        wave_find256(hist + grp * 256, need - above, &bb, &rr);
        b = grp * 256 + (int)bb;
        above = need - rr;
        break;
      }
      above += c;
    }
    if (tid == 0) { sh[0] = b; sh[1] = (int)(need - above); }
  }
  __syncthreads();
  const int tb = sh[0];
  need = (uint32_t)sh[1];
  __syncthreads();

  // The keys whose bin is tb form one contiguous key range [lo, hi] (the
  // bin function is monotone in the key between key(-inf) and key(+inf));
  // one thread finds its ends by bisection.
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
    sh[2] = (int)a;
    sh[3] = (int)c;
  }
  __syncthreads();
  const uint32_t lo = (uint32_t)sh[2], hi = (uint32_t)sh[3];
  __syncthreads();
  // four 8-bit radix passes over the offsets k - lo of the keys in [lo, hi]
  uint32_t prefix = 0, pmask = 0;
  for (int p = 0; p < 4; ++p) {
    const int s = 24 - 8 * p;
    for (int i = tid; i < 256; i += NT) hist[i] = 0u;
    __syncthreads();
    for (int i = tid; i < G; i += NT) {
      const uint32_t k = score_key(srow[i]);
      const uint32_t off = k - lo;
      if (k >= lo && k <= hi && (off & pmask) == prefix) atomicAdd(&hist[(off >> s) & 255u], 1u);
    }
    __syncthreads();
    uint32_t d;
    block_find256(hist, need, sh, &d, &need);
    prefix |= d << s;
    pmask |= 255u << s;
  }
  *take_eq = need;
  return lo + prefix;
}

// Wave-level search of a 4,096-bin histogram for the bin holding the
// need-th largest element: count(bins > b) < need <= count(bins >= b).
// Lane l first sums the 64 bins of chunk 63 - l (lane 0: the top chunk),
// then each lane takes one bin of the chosen chunk.
__device__ __forceinline__ void wave_find4096(const uint32_t* hist, uint32_t need, uint32_t* bin,
                                              uint32_t* rem) {
  const int lane = threadIdx.x & (kWave - 1);
  const uint4* h4 = reinterpret_cast<const uint4*>(hist) + 16 * (63 - lane);
  uint32_t part = 0u;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const uint4 v = h4[q];
    part += (v.x + v.y) + (v.z + v.w);
  }
  uint32_t incl = wave_incl_scan(part);
  uint64_t m = __ballot(incl - part < need && need <= incl);
  int src = m ? __ffsll((unsigned long long)m) - 1 : 0;
  const uint32_t need2 = need - ((uint32_t)__shfl((int)incl, src, kWave) -
                                 (uint32_t)__shfl((int)part, src, kWave));
  const int chunk = 63 - src;
  const uint32_t c = hist[64 * chunk + 63 - lane];
  incl = wave_incl_scan(c);
  m = __ballot(incl - c < need2 && need2 <= incl);
  src = m ? __ffsll((unsigned long long)m) - 1 : 0;
  *bin = (uint32_t)(64 * chunk + 63 - src);
  *rem = need2 - ((uint32_t)__shfl((int)incl, src, kWave) - (uint32_t)__shfl((int)c, src, kWave));
}

// The need-th largest of M candidate keys per thread (0 = empty slot), all
// within [kmin, kmax], and how many copies of it are taken: radix passes of
// up to 12 bits over the offsets key - kmin (two passes for spans up to
// 2^24), with a 4,096-bin LDS histogram.
template <int NT, int M>
__device__ uint32_t wide_threshold(const uint32_t (&key)[M], uint32_t kmin, uint32_t kmax,
                                   uint32_t need, uint32_t* hist, int* sh, uint32_t* take_eq) {
  const int tid = threadIdx.x;
  const uint32_t span = kmax >= kmin ? kmax - kmin : 0u;
  int nbits = span ? 32 - __clz(span) : 0;
  uint32_t prefix = 0, pmask = 0;
  while (nbits > 0) {
    const int sft = nbits > 12 ? nbits - 12 : 0;
    const uint32_t dmask = (1u << (nbits - sft)) - 1u;
    for (int i = tid; i < 4096; i += NT) hist[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const uint32_t off = key[m] - kmin;
      if (key[m] && (off & pmask) == prefix) atomicAdd(&hist[(off >> sft) & dmask], 1u);
    }
    __syncthreads();
    if (tid < kWave) {
      uint32_t b, r;
      wave_find4096(hist, need, &b, &r);
      if (tid == 0) { sh[0] = (int)b; sh[1] = (int)r; }
    }
    __syncthreads();
    prefix |= (uint32_t)sh[0] << sft;
    need = (uint32_t)sh[1];
    pmask |= dmask << sft;
    nbits = sft;
  }
  *take_eq = need;
  return kmin + prefix;
}

// The groups marked in selmap, plus the first take_eq (in index order) of
// those marked in eqmap, written in ascending order to orow[0, K).  Thread
// t owns bitmap words [WPT t, WPT t + WPT); two block scans place them.
template <int NT, int WPT>
__device__ __forceinline__ void emit_selection(const uint32_t* selmap, const uint32_t* eqmap,
                                               int nwords, uint32_t take_eq, int K,
                                               int32_t* orow, uint32_t* tmp) {
  const int tid = threadIdx.x;
  uint32_t sw[WPT], ew[WPT];
  uint32_t n_eq = 0;
#pragma unroll
  for (int i = 0; i < WPT; ++i) {
    const int w = tid * WPT + i;
    sw[i] = w < nwords ? selmap[w] : 0u;
    ew[i] = w < nwords ? eqmap[w] : 0u;
    n_eq += (uint32_t)__popc(ew[i]);
  }
  uint32_t eq_before = block_excl_scan<NT>(n_eq, tmp);
  uint32_t n_sel = 0;
#pragma unroll
  for (int i = 0; i < WPT; ++i) {
    uint32_t w = ew[i];
    while (w) {
      const uint32_t bit = w & (~w + 1u);
      if (eq_before < take_eq) sw[i] |= bit;
      ++eq_before;
      w ^= bit;
    }
    n_sel += (uint32_t)__popc(sw[i]);
  }
  uint32_t pos = block_excl_scan<NT>(n_sel, tmp);
#pragma unroll
  for (int i = 0; i < WPT; ++i) {
    uint32_t w = sw[i];
    while (w) {
      const int b = __ffs(w) - 1;
      if (pos < (uint32_t)K) orow[pos] = 32 * (tid * WPT + i) + b;
      ++pos;
      w &= w - 1u;
    }
  }
}

// ---------------------------------------------------------------------------
// extract: one workgroup per (slice, row), a row's slices on one XCD

__global__ __launch_bounds__(kExtractThreads) void topk_extract_kernel(
    const float* __restrict__ scores, int gstride, const int32_t* __restrict__ row_len,
    int first_pos, int max_ctx, int K, uint32_t* __restrict__ cand_val,
    uint16_t* __restrict__ cand_idx, int32_t* __restrict__ cand_cnt,
    const float* __restrict__ samples) {
  static_assert(kSample == kTopkSamples, "one sample layout");
  constexpr int NT = kExtractThreads, NW = NT / kWave;
  constexpr int E4 = kSlice / (4 * NT);  // float4 chunks per thread
  constexpr int kCW = kSliceCap / NW;    // slots per wave
  __shared__ __attribute__((aligned(16))) uint32_t hist[256];
  __shared__ uint32_t sval[kSliceCap];
  __shared__ uint16_t sidx[kSliceCap];
  __shared__ uint32_t wcnt[NW];
  __shared__ uint32_t wmax[NW];
  __shared__ float sguess;

  // workgroup b -> row b % n_rows, slice b / n_rows: workgroups are dealt to
  // the XCDs round-robin, so with 8 | n_rows a row's slices share the XCD of
  // its finish workgroup (row r is finish workgroup r) and the finish finds
  // more of the candidates in that XCD's L2 (measured: 196.35 -> 195.45 us
  // per decode step of 8 x 262,144 tokens)
  const int n_rows = gridDim.x / ((gstride + kSlice - 1) / kSlice);
  const int slice = blockIdx.x / n_rows, row = blockIdx.x - slice * n_rows;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const size_t slot0 = ((size_t)row * kMaxSlices + slice) * kSliceCap;
  const int g0 = slice * kSlice;
  const float* srow = scores + (size_t)row * gstride;

  // Slice loads and the scoring kernel's sample are issued before the row
  // length is known (both stay inside their rows), so their latency
  // overlaps the length load; entries past the row's groups are masked
  // once it is.
  uint32_t v[4 * E4];
#pragma unroll
  for (int e = 0; e < E4; ++e) {
    const int c0 = g0 + 4 * (e * NT + tid);
    if (((reinterpret_cast<uintptr_t>(srow) & 15u) == 0u) && c0 + 3 < gstride) {
      const float4 f = *reinterpret_cast<const float4*>(srow + c0);
      v[4 * e] = __float_as_uint(f.x); v[4 * e + 1] = __float_as_uint(f.y);
      v[4 * e + 2] = __float_as_uint(f.z); v[4 * e + 3] = __float_as_uint(f.w);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        v[4 * e + j] = c0 + j < gstride ? __float_as_uint(srow[c0 + j]) : 0x7FC00000u;
    }
  }
  float sv[8];
  if (samples && wid == 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) sv[i] = samples[(size_t)row * kSample + lane + kWave * i];
  }
  const int L = row_len ? row_len[row] : first_pos + row + 1;
  int G = (L >= 0 && L <= max_ctx) ? L / kRatio : 0;
  if (G > gstride) G = gstride;
  int32_t* info = cand_cnt + (size_t)(row * kMaxSlices + slice) * kInfo;
  if (G <= K || g0 >= G) {  // finish handles the row alone / empty slice
    if (tid == 0) { info[0] = 0; info[1] = 0; info[2] = 0; }
    return;
  }
#pragma unroll
  for (int e = 0; e < E4; ++e)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (g0 + 4 * (e * NT + tid) + j >= G) v[4 * e + j] = 0x7FC00000u;  // NaN: never kept

  if (wid == 0) {
    uint32_t sk[8];
    const bool have = samples && G >= kSample;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int si = (int)(((long long)(lane + kWave * i) * G) / kSample);
      sk[i] = score_key(have ? sv[i] : srow[si]);
    }
    const int r0 = (int)(((long long)kSample * K + G - 1) / G);
    int r = r0 + 4 * (int)ceilf(sqrtf((float)r0)) + 4;
    if (r > kSample) r = kSample;
    const uint32_t gk = wave_select_rth(sk, (uint32_t)r, hist);
    if (lane == 0) {
      sguess = key_value(gk);
      info[2] = (int32_t)gk;
    }
  }
  __syncthreads();
  const float guess = sguess;

  // keep scores >= guess, each wave in its own region, in order
  uint32_t run = 0;
  float kmx_f = -INFINITY;
#pragma unroll
  for (int e = 0; e < 4 * E4; ++e) {
    const bool pred = __uint_as_float(v[e]) >= guess;
    const uint64_t mask = __ballot(pred);
    const uint32_t pos = run + __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                         __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
    if (pred && pos < (uint32_t)kCW) {
      sval[wid * kCW + pos] = v[e];
      sidx[wid * kCW + pos] = (uint16_t)(g0 + 4 * ((e / 4) * NT + tid) + (e % 4));
    }
    if (pred) kmx_f = fmaxf(kmx_f, __uint_as_float(v[e]));  // kept scores are not NaN
    run += (uint32_t)__popcll(mask);
  }
  const uint32_t kmx = wave_max_u32(run ? score_key(kmx_f) : 0u);  // score_key is monotone
  if (lane == 0) { wcnt[wid] = run; wmax[wid] = kmx; }
  __syncthreads();
  uint32_t before = 0, total = 0;
  bool over = false;
  for (int w = 0; w < NW; ++w) {
    if (w < wid) before += wcnt[w];
    total += wcnt[w];
    over |= wcnt[w] > (uint32_t)kCW;
  }
  if (!over) {
    for (uint32_t i = lane; i < wcnt[wid]; i += kWave) {
      cand_val[slot0 + before + i] = sval[wid * kCW + i];
      cand_idx[slot0 + before + i] = sidx[wid * kCW + i];
    }
  }
  if (tid == 0) {
    uint32_t m = 0u;
    for (int w = 0; w < NW; ++w) m = max(m, wmax[w]);
    info[0] = over ? kSliceCap + 1 : (int)total;
    info[1] = (int32_t)m;
  }
}

// ---------------------------------------------------------------------------
// finish: one workgroup per long row, over the candidates its slices kept

__global__ __launch_bounds__(kFinishThreads) void topk_finish_kernel(
    const float* __restrict__ scores, int gstride, const int32_t* __restrict__ row_len,
    int first_pos, int max_ctx, int K, const uint32_t* __restrict__ cand_val,
    const uint16_t* __restrict__ cand_idx, const int32_t* __restrict__ cand_cnt,
    int32_t* __restrict__ out) {
  constexpr int NT = kFinishThreads, NW = NT / kWave;
  constexpr int MC = kMaxSlices;        // slot row m of thread t: slice m, slot t
  constexpr int kW = kMaxGroups / 32;   // bitmap words
  static_assert(kSliceCap == NT, "one slice per slot row");
  __shared__ __attribute__((aligned(16))) uint32_t hist[kBins];
  __shared__ uint32_t selmap[kW];
  __shared__ uint32_t eqmap[kW];
  __shared__ uint32_t tmp[2 * NW + 1];
  __shared__ float red[2 * NW];
  __shared__ int sh[4];
  constexpr int kBinRank = kWave;  // boundary-bin candidates ranked directly
  __shared__ uint32_t bin_key[kBinRank];
  __shared__ uint32_t bin_grp[kBinRank];

  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  // Candidate slots and the slices' records are fetched first, before the
  // row length is known (every slot lies inside the workspace), so their
  // latency overlaps the length load.
  uint32_t ck[MC], cg[MC], kmx[MC];
  int cnt[MC];
  const size_t base = (size_t)row * kMaxSlices * kSliceCap;
#pragma unroll
  for (int m = 0; m < MC; ++m) {
    cnt[m] = cand_cnt[(size_t)(row * kMaxSlices + m) * kInfo];
    kmx[m] = (uint32_t)cand_cnt[(size_t)(row * kMaxSlices + m) * kInfo + 1];
    ck[m] = cand_val[base + m * NT + tid];
    cg[m] = cand_idx[base + m * NT + tid];
  }
  // the guess (slice 0 always derives it): every candidate key is >= gk
  const uint32_t gk = (uint32_t)cand_cnt[(size_t)row * kMaxSlices * kInfo + 2];
  const int L = row_len ? row_len[row] : first_pos + row + 1;
  int G = (L >= 0 && L <= max_ctx) ? L / kRatio : 0;
  if (G > gstride) G = gstride;
  int32_t* orow = out + (size_t)row * K;
  if (G <= K) {  // every complete group is kept
    for (int i = tid; i < K; i += NT) orow[i] = (i < G) ? i : -1;
    return;
  }
  const float* srow = scores + (size_t)row * gstride;
  const int nwords = (G + 31) / 32;
  for (int i = tid; i < nwords; i += NT) { selmap[i] = 0u; eqmap[i] = 0u; }

  const int n_slices = (G + kSlice - 1) / kSlice;
  bool ok = true;
  uint32_t C = 0;
#pragma unroll
  for (int m = 0; m < MC; ++m) {
    cnt[m] = m < n_slices ? cnt[m] : 0;
    ok &= cnt[m] <= kSliceCap;
    C += (uint32_t)cnt[m];
  }
  ok &= C >= (uint32_t)K;
  uint32_t T = 0, take_eq = 0;
  if (ok) {
    uint32_t kmax = 0u;
#pragma unroll
    for (int m = 0; m < MC; ++m) {
      ck[m] = tid < cnt[m] ? score_key(__uint_as_float(ck[m])) : 0u;
      kmax = max(kmax, cnt[m] > 0 ? kmx[m] : 0u);
    }
    // One 12-bit radix pass over the top bits of key - gk finds the bin of
    // the K-th key and how many of that bin's keys are taken; the bin
    // rarely holds more than a few candidates (2 - 7 in 8 x 65,536 N(0,1)
    // scores), so one wavefront ranks them by (key desc, index asc) instead
    // of a second pass.  More than kBinRank of them: the full radix
    // threshold below.
    bool done = false;
    const uint32_t span = kmax >= gk ? kmax - gk : 0u;
    const int nbits = span ? 32 - __clz(span) : 0;
    if (nbits > 12) {
      const int sft = nbits - 12;
      for (int i = tid; i < 4096; i += NT) hist[i] = 0u;
      if (tid == 0) sh[2] = 0;
      __syncthreads();
#pragma unroll
      for (int m = 0; m < MC; ++m)
        if (ck[m]) atomicAdd(&hist[((ck[m] - gk) >> sft) & 4095u], 1u);
      __syncthreads();
      if (tid < kWave) {
        uint32_t b, r;
        wave_find4096(hist, (uint32_t)K, &b, &r);
        if (tid == 0) { sh[0] = (int)b; sh[1] = (int)r; }
      }
      __syncthreads();
      const uint32_t bb = (uint32_t)sh[0], rem = (uint32_t)sh[1];
#pragma unroll
      for (int m = 0; m < MC; ++m) {
        if (ck[m] && ((ck[m] - gk) >> sft) == bb) {
          const int pos = atomicAdd(&sh[2], 1);
          if (pos < kBinRank) { bin_key[pos] = ck[m]; bin_grp[pos] = cg[m]; }
        }
      }
      __syncthreads();
      const int nm = sh[2];
      if (nm <= kBinRank) {
#pragma unroll
        for (int m = 0; m < MC; ++m)
          if (ck[m] && ((ck[m] - gk) >> sft) > bb) atomicOr(&selmap[cg[m] >> 5], 1u << (cg[m] & 31));
        if (tid < nm) {
          const uint32_t mk = bin_key[tid], mg = bin_grp[tid];
          uint32_t rank = 0;
          for (int j = 0; j < nm; ++j) {
            const uint32_t kj = bin_key[j];
            rank += (kj > mk || (kj == mk && bin_grp[j] < mg)) ? 1u : 0u;
          }
          if (rank < rem) atomicOr(&selmap[mg >> 5], 1u << (mg & 31));
        }
        done = true;
      }
    }
    if (!done) {
      T = wide_threshold<NT, MC>(ck, gk, kmax, (uint32_t)K, hist, sh, &take_eq);
#pragma unroll
      for (int m = 0; m < MC; ++m)
        if (ck[m] >= T && ck[m]) atomicOr(ck[m] > T ? &selmap[cg[m] >> 5] : &eqmap[cg[m] >> 5],
                                          1u << (cg[m] & 31));
    }
  } else {
    // the pruning guess missed: exact ranking of the whole row
    T = exact_threshold_stream<NT>(srow, G, (uint32_t)K, hist, red, sh, &take_eq);
    for (int i = tid; i < G; i += NT) {
      const uint32_t k = score_key(srow[i]);
      if (k >= T) atomicOr(k > T ? &selmap[i >> 5] : &eqmap[i >> 5], 1u << (i & 31));
    }
  }
  __syncthreads();

  emit_selection<NT, kW / NT>(selmap, eqmap, nwords, take_eq, K, orow, tmp);
}

// ---------------------------------------------------------------------------
// row: one workgroup per short row (thousands of them in a prefill chunk).
// Ranking every key of the row costs several ALU operations per key and
// pass, so the row is pruned first, as the extract step prunes a slice:
// the guess is the exact r-th largest of 512 evenly spaced sample keys,
// every key >= guess is compacted into LDS (about K + 4 sqrt(K) of the
// row), and only those are ranked.  If a wave's candidates overflow its
// LDS region or fewer than K survive, the whole row is ranked instead.

// The need-th largest of the candidate keys (all >= kmin, at most kmax;
// 0 = empty slot; only the first `active` slots of each thread can be
// occupied) and how many copies of it are taken: radix passes of 8 bits
// over the offsets key - kmin.
template <int NT, int M>
__device__ uint32_t pruned_threshold(const uint32_t (&key)[M], int active, uint32_t kmin,
                                     uint32_t kmax, uint32_t need, uint32_t* hist, int* sh,
                                     uint32_t* take_eq) {
  const int tid = threadIdx.x;
  const uint32_t span = kmax - kmin;
  int nbits = span ? 32 - __clz(span) : 0;
  uint32_t prefix = 0, pmask = 0;
  while (nbits > 0) {
    const int sft = nbits > 8 ? nbits - 8 : 0;
    const uint32_t dmask = (1u << (nbits - sft)) - 1u;
    for (int i = tid; i < 256; i += NT) hist[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int m = 0; m < M; ++m) {
      if (m < active) {
        const uint32_t off = key[m] - kmin;
        if (key[m] && (off & pmask) == prefix) atomicAdd(&hist[(off >> sft) & dmask], 1u);
      }
    }
    __syncthreads();
    uint32_t d;
    block_find256(hist, need, sh, &d, &need);
    prefix |= d << sft;
    pmask |= dmask << sft;
    nbits = sft;
  }
  *take_eq = need;
  return kmin + prefix;
}

template <int NT, int kMaxG>
__global__ __launch_bounds__(NT) void topk_row_kernel(const float* __restrict__ scores,
                                                      int gstride,
                                                      const int32_t* __restrict__ row_len,
                                                      int first_pos, int max_ctx, int K,
                                                      int32_t* __restrict__ out) {
  constexpr int NW = NT / kWave;
  constexpr int E = kMaxG / (4 * NT);   // 16-byte chunks per thread
  constexpr int M = 4 * E;              // keys per thread: key 4e + c is group 4 (e NT + t) + c
  constexpr int kW = kMaxG / 32 > NT ? kMaxG / 32 : NT;  // bitmap words
  static_assert(kMaxG <= 65536 && M <= 32, "16-bit group ids, one mask bit per key");
  constexpr int kCW = kRowCap / NW;     // candidate slots per wave
  constexpr int MC = kRowCap / NT;      // candidate slots per thread
  __shared__ __attribute__((aligned(16))) uint32_t hist[256];
  __shared__ uint32_t selmap[kW];
  __shared__ uint32_t eqmap[kW];
  __shared__ uint32_t cval[kRowCap];
  __shared__ uint16_t cidx[kRowCap];
  __shared__ uint32_t wcnt[NW];
  __shared__ uint32_t tmp[2 * NW + 1];
  __shared__ float red[2 * NW];
  __shared__ int sh[4];

  const int row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const int L = row_len ? row_len[row] : first_pos + row + 1;
  int G = (L >= 0 && L <= max_ctx) ? L / kRatio : 0;
  if (G > gstride) G = gstride;
  int32_t* orow = out + (size_t)row * K;
  if (G <= K) {  // every complete group is kept
    for (int i = tid; i < K; i += NT) orow[i] = (i < G) ? i : -1;
    return;
  }
  // the row's scores (addresses clamped into the row instead of branching
  // per lane; entries past its groups are masked below) and, for wave 0,
  // the sample, all issued together
  const float* srow = scores + (size_t)row * gstride;
  uint32_t ck[M];
  if ((gstride & 3) == 0 && (reinterpret_cast<uintptr_t>(scores) & 15u) == 0u) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float4 f = *reinterpret_cast<const float4*>(srow + min(4 * (e * NT + tid), gstride - 4));
      ck[4 * e] = __float_as_uint(f.x); ck[4 * e + 1] = __float_as_uint(f.y);
      ck[4 * e + 2] = __float_as_uint(f.z); ck[4 * e + 3] = __float_as_uint(f.w);
    }
  } else {
#pragma unroll
    for (int j = 0; j < M; ++j)
      ck[j] = __float_as_uint(srow[min(4 * ((j >> 2) * NT + tid) + (j & 3), gstride - 1)]);
  }
  float sv[8];
  if (wid == 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) sv[i] = srow[(int)(((long long)(lane + kWave * i) * G) / kSample)];
  }
  const int nwords = (G + 31) / 32;
  for (int i = tid; i < nwords; i += NT) { selmap[i] = 0u; eqmap[i] = 0u; }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int lim = G - 4 * (e * NT + tid);  // keys of chunk e below G
#pragma unroll
    for (int c = 0; c < 4; ++c)
      ck[4 * e + c] = c < lim ? score_key(__uint_as_float(ck[4 * e + c])) : 0u;
  }
  if (wid == 0) {
    uint32_t sk[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) sk[i] = score_key(sv[i]);
    const int r0 = (int)(((long long)kSample * K + G - 1) / G);
    int r = r0 + 4 * (int)ceilf(sqrtf((float)r0)) + 4;
    if (r > kSample) r = kSample;
    const uint32_t gk = wave_select_rth(sk, (uint32_t)r, hist);
    if (lane == 0) { sh[0] = (int)gk; sh[3] = 0; }
  }
  __syncthreads();
  const uint32_t gk = (uint32_t)sh[0];
  // keys >= guess, each wave into its own region, in order; the largest
  // candidate key bounds the radix passes
  uint32_t run = 0, kmax = 0u;
#pragma unroll
  for (int j = 0; j < M; ++j) {
    const bool pred = ck[j] >= gk && ck[j] != 0u;
    const uint64_t bm = __ballot(pred);
    const uint32_t pos = run + __builtin_amdgcn_mbcnt_hi((uint32_t)(bm >> 32),
                                                         __builtin_amdgcn_mbcnt_lo((uint32_t)bm, 0u));
    if (pred && pos < (uint32_t)kCW) {
      cval[wid * kCW + pos] = ck[j];
      cidx[wid * kCW + pos] = (uint16_t)(4 * ((j >> 2) * NT + tid) + (j & 3));
    }
    if (pred) kmax = max(kmax, ck[j]);
    run += (uint32_t)__popcll(bm);
  }
  kmax = wave_max_u32(kmax);
  if (lane == 0) {
    wcnt[wid] = run;
    atomicMax(reinterpret_cast<uint32_t*>(&sh[3]), kmax);
  }
  __syncthreads();
  uint32_t total = 0, most = 0;
  bool over = false;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    total += wcnt[w];
    most = max(most, wcnt[w]);
    over |= wcnt[w] > (uint32_t)kCW;
  }
  uint32_t T = 0, take_eq = 0;
  if (!over && total >= (uint32_t)K) {
    // candidate m of this thread is slot row m / NW of wave region m % NW;
    // only the first `active` slot rows of a region can be occupied
    const int active = (int)((most + NT - 1) / NT);
    auto slot = [&](int m) { return (m % NW) * kCW + (m / NW) * NT + tid; };
    uint32_t c[MC];
#pragma unroll
    for (int m = 0; m < MC; ++m)
      c[m] = m / NW < active && (uint32_t)((m / NW) * NT + tid) < wcnt[m % NW] ? cval[slot(m)] : 0u;
    T = pruned_threshold<NT, MC>(c, active * NW, gk, (uint32_t)sh[3], (uint32_t)K, hist, sh,
                                 &take_eq);
#pragma unroll
    for (int m = 0; m < MC; ++m) {
      if (c[m] >= T && c[m]) {
        const uint32_t g = cidx[slot(m)];
        atomicOr(c[m] > T ? &selmap[g >> 5] : &eqmap[g >> 5], 1u << (g & 31));
      }
    }
  } else {
    // the guess missed: rank the whole row
    T = row_threshold<NT, M>(ck, (uint32_t)K, hist, red, sh, &take_eq);
#pragma unroll
    for (int j = 0; j < M; ++j) {
      const uint32_t g = (uint32_t)(4 * ((j >> 2) * NT + tid) + (j & 3));
      if (ck[j] >= T && ck[j]) atomicOr(ck[j] > T ? &selmap[g >> 5] : &eqmap[g >> 5], 1u << (g & 31));
    }
  }
  __syncthreads();
  emit_selection<NT, kW / NT>(selmap, eqmap, nwords, take_eq, K, orow, tmp);
}

// ---------------------------------------------------------------------------
// wave: one wavefront per row of up to 64 M groups (short decode contexts,
// early prefill queries), four rows per workgroup.  Lane l owns groups
// [M l, M l + M): the exact K-th key comes from four radix passes over a
// histogram owned by the wave, and the selection is emitted from per-lane
// bit masks with wave scans, so no barrier is involved.

template <int M>
__global__ __launch_bounds__(kWave * 4) void topk_wave_kernel(const float* __restrict__ scores,
                                                             int gstride,
                                                             const int32_t* __restrict__ row_len,
                                                             int first_pos, int max_ctx, int n_rows,
                                                             int K, int32_t* __restrict__ out) {
  static_assert(M % 4 == 0 && M <= 64, "groups per lane");
  __shared__ __attribute__((aligned(16))) uint32_t hist_all[4][256];
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  const int row = blockIdx.x * 4 + wid;
  if (row >= n_rows) return;  // whole wavefronts leave; nothing below synchronises the block
  uint32_t* hist = hist_all[wid];
  const int L = row_len ? row_len[row] : first_pos + row + 1;
  int G = (L >= 0 && L <= max_ctx) ? L / kRatio : 0;
  if (G > gstride) G = gstride;
  int32_t* orow = out + (size_t)row * K;
  if (G <= K) {  // every complete group is kept
    for (int i = lane; i < K; i += kWave) orow[i] = (i < G) ? i : -1;
    return;
  }
  const float* srow = scores + (size_t)row * gstride;
  const int g0 = M * lane;
  uint32_t key[M];
  if ((gstride & 3) == 0 && (reinterpret_cast<uintptr_t>(scores) & 15u) == 0u) {
#pragma unroll
    for (int e = 0; e < M / 4; ++e) {
      // clamped into the row; entries past G are masked below
      const float4 f = *reinterpret_cast<const float4*>(srow + min(g0 + 4 * e, gstride - 4));
      key[4 * e] = __float_as_uint(f.x); key[4 * e + 1] = __float_as_uint(f.y);
      key[4 * e + 2] = __float_as_uint(f.z); key[4 * e + 3] = __float_as_uint(f.w);
    }
  } else {
#pragma unroll
    for (int j = 0; j < M; ++j) key[j] = __float_as_uint(srow[min(g0 + j, gstride - 1)]);
  }
#pragma unroll
  for (int j = 0; j < M; ++j) key[j] = g0 + j < G ? score_key(__uint_as_float(key[j])) : 0u;
  const uint32_t T = wave_select_span<M>(key, (uint32_t)K, hist);
  // groups above T are taken; of those equal to T, the lowest-indexed ones
  // up to K in all
  uint64_t gt = 0u, eq = 0u;
#pragma unroll
  for (int j = 0; j < M; ++j) {
    gt |= (key[j] > T) ? 1ull << j : 0ull;
    eq |= (key[j] == T && key[j] != 0u) ? 1ull << j : 0ull;
  }
  const uint32_t n_gt = (uint32_t)__popcll(gt), n_eq = (uint32_t)__popcll(eq);
  const uint32_t gt_incl = wave_incl_scan(n_gt), eq_incl = wave_incl_scan(n_eq);
  const uint32_t take_eq = (uint32_t)K - (uint32_t)__shfl((int)gt_incl, kWave - 1, kWave);
  uint32_t eq_before = eq_incl - n_eq;
  uint64_t sel = gt;
  for (uint64_t w = eq; w && eq_before < take_eq; w &= w - 1u, ++eq_before) sel |= w & (~w + 1u);
  const uint32_t n_sel = (uint32_t)__popcll(sel);
  uint32_t pos = wave_incl_scan(n_sel) - n_sel;
  for (uint64_t w = sel; w; w &= w - 1u, ++pos)
    if (pos < (uint32_t)K) orow[pos] = g0 + __ffsll((unsigned long long)w) - 1;
}

}  // namespace

size_t topk_workspace_bytes(int n_rows, int gstride) {
  if (gstride <= kDirect) return 0;
  const size_t slots = (size_t)n_rows * kMaxSlices * kSliceCap;
  return slots * sizeof(uint32_t) + slots * sizeof(uint16_t) +
         (size_t)n_rows * kMaxSlices * kInfo * sizeof(int32_t) + 3 * 256;
}

hipError_t launch_topk(const float* scores, int gstride, int n_rows, const int32_t* row_len,
                       int first_pos, int max_ctx, int K, int32_t* out, void* ws,
                       hipStream_t stream, const float* samples) {
  if (n_rows <= 0) return hipSuccess;
  if (gstride > kMaxGroups) return hipErrorInvalidValue;
  if (gstride <= kWaveRow) {
    // short rows: one wavefront each, 32 groups per lane
    hipLaunchKernelGGL((topk_wave_kernel<kWaveRow / kWave>), dim3((n_rows + 3) / 4),
                       dim3(kWave * 4), 0, stream, scores, gstride, row_len, first_pos, max_ctx,
                       n_rows, K, out);
    return hipGetLastError();
  }
  if (gstride <= kShort) {
    // many short rows (prefill): small workgroups, several rows per CU
    hipLaunchKernelGGL((topk_row_kernel<kShortThreads, kShort>), dim3(n_rows),
                       dim3(kShortThreads), 0, stream, scores, gstride, row_len, first_pos, max_ctx,
                       K, out);
    return hipGetLastError();
  }
  if (gstride <= kDirect) {
    // a few longer rows: twice the threads, the same 32 keys each
    hipLaunchKernelGGL((topk_row_kernel<2 * kShortThreads, kDirect>), dim3(n_rows),
                       dim3(2 * kShortThreads), 0, stream, scores, gstride, row_len, first_pos,
                       max_ctx, K, out);
    return hipGetLastError();
  }
  if (!ws) return hipErrorInvalidValue;
  const size_t slots = (size_t)n_rows * kMaxSlices * kSliceCap;
  char* p = reinterpret_cast<char*>(ws);
  uint32_t* cval = reinterpret_cast<uint32_t*>(p);
  p += (slots * sizeof(uint32_t) + 255) / 256 * 256;
  uint16_t* cidx = reinterpret_cast<uint16_t*>(p);
  p += (slots * sizeof(uint16_t) + 255) / 256 * 256;
  int32_t* ccnt = reinterpret_cast<int32_t*>(p);
  const int n_slices = (gstride + kSlice - 1) / kSlice;
  hipLaunchKernelGGL(topk_extract_kernel, dim3(n_slices * n_rows), dim3(kExtractThreads), 0,
                     stream, scores, gstride, row_len, first_pos, max_ctx, K, cval, cidx, ccnt,
                     samples);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_finish_kernel,
                     dim3(n_rows), dim3(kFinishThreads), 0, stream, scores, gstride, row_len,
                     first_pos, max_ctx, K, cval, cidx, ccnt, out);
  return hipGetLastError();
}

}  // namespace qsa
