// index_score.hip — indexer scoring at decode: an fp32 GEMV per query row
// over the request's paged compressed keys k̂.
//
// Per complete group g of the row (the C4 groups of the "QSA in brief"
// section of the Qwen3.8-27B QSA model card; the scoring form is the
// library's stated reading, since the pages give none):
//   score[g] = sum_h w[h] * max(0, sum_d q[h,d] * khat[g,h,d])
//
// The work is a stream over k̂ (2 KiB per group, 0.5 flop per byte), so the
// kernel is built for HBM bandwidth, not arithmetic:
//   - one wavefront consumes one 32 KiB k̂ page (16 groups) with fully
//     coalesced, non-temporal 16-byte loads (k̂ is read once per step):
//     lane l reads float4 #l of each 1 KiB half of a group, i.e. heads l/16
//     and 4 + l/16, dims 4*(l%16) .. +3;
//   - each lane keeps the matching 8 query values and 2 weights in
//     registers for the whole launch;
//   - per-head dot products finish with DPP row reductions (a DPP row is
//     exactly the 16 lanes that hold one head);
//   - the 16 group scores are transposed so lanes 0..15 own one group each,
//     summed across the 4 rows with two cross-row shuffles and stored as
//     one 64-byte coalesced write.
#include "qsa_device.h"
#include "qsa_launch.h"

namespace qsa {
namespace {

constexpr int kScoreThreads = 128;  // 2 waves, one k̂ page each
constexpr int kScoreWaves = kScoreThreads / kWave;
// One page per wavefront and two wavefronts per workgroup: the grid (8 rows
// x 4,096 pages = 16,384 workgroups at the longest context) drains in fine
// steps, and each wave's chain of dependent loads (row length, page id, k̂)
// is paid once.
constexpr int kPagesPerWave = 1;

__device__ __forceinline__ float dot4(float4 a, float4 b) {
  return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
}

__global__ __launch_bounds__(kScoreThreads) void index_score_gemv_kernel(
    const float* __restrict__ khat, const int32_t* __restrict__ page_table, int max_pages,
    int num_pages, const int32_t* __restrict__ row_req, const int32_t* __restrict__ row_len,
    int req0, int first_pos, int max_ctx, const float* __restrict__ q_idx,
    const float* __restrict__ w_idx, float* __restrict__ scores, int gstride,
    float* __restrict__ samples) {
  // rows carry their own (request, length); with row_req null, row r uses
  // page-table row r; with both null, rows are the consecutive queries of
  // request req0 starting at position first_pos
  const int row = blockIdx.y;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int L = row_len ? row_len[row] : first_pos + row + 1;
  const int G = (L >= 0 && L <= max_ctx) ? L / kRatio : 0;
  const int req = row_req ? row_req[row] : (row_len ? row : req0);

  const int hA = lane >> 4, hB = 4 + (lane >> 4), d0 = 4 * (lane & 15);
  const float* qrow = q_idx + (size_t)row * kGroupFloats;
  float4 qa = *reinterpret_cast<const float4*>(qrow + hA * kIdxDim + d0);
  float4 qb = *reinterpret_cast<const float4*>(qrow + hB * kIdxDim + d0);
  const float wa = w_idx[(size_t)row * kIdxHeads + hA];
  const float wb = w_idx[(size_t)row * kIdxHeads + hB];

  float* srow = scores + (size_t)row * gstride;
  const int row_pages = (gstride + kGroupsPerPage - 1) / kGroupsPerPage;
  const int* pt = page_table + (size_t)req * max_pages;

  for (int i = 0; i < kPagesPerWave; ++i) {
    const int page = blockIdx.x * kScoreWaves * kPagesPerWave + i * kScoreWaves + wave;
    if (page >= row_pages) break;
    const int g0 = page * kGroupsPerPage;
    float sc = -INFINITY;
    if (g0 < G) {
      const int phys = pt[page];
      if (phys >= 0 && phys < num_pages) {
        const float4* base =
            reinterpret_cast<const float4*>(khat + (size_t)phys * kGroupsPerPage * kGroupFloats);
        float v[kGroupsPerPage];
#pragma unroll
        for (int g = 0; g < kGroupsPerPage; ++g) {
          float4 x0 = stream_load(base + g * 128 + lane);
          float4 x1 = stream_load(base + g * 128 + 64 + lane);
          float p0 = row16_sum(dot4(x0, qa));
          float p1 = row16_sum(dot4(x1, qb));
          v[g] = wa * fmaxf(p0, 0.0f) + wb * fmaxf(p1, 0.0f);
        }
        // lane l keeps its row's partial of group l % 16
        float keep = v[0];
#pragma unroll
        for (int g = 1; g < kGroupsPerPage; ++g) keep = ((lane & 15) == g) ? v[g] : keep;
        keep += __shfl_xor(keep, 16, kWave);
        keep += __shfl_xor(keep, 32, kWave);
        if (g0 + (lane & 15) < G) sc = keep + 0.0f;  // -0 -> +0
      }
    }
    if (lane < kGroupsPerPage && g0 + lane < gstride) {
      srow[g0 + lane] = sc;
      // group g is sample i when floor(i * G / n) = g, i.e. i = ceil(g * n / G)
      const int g = g0 + lane;
      if (samples && G >= kTopkSamples && g < G) {
        const int i = (int)(((long long)g * kTopkSamples + G - 1) / G);
        if (i < kTopkSamples && (int)(((long long)i * G) / kTopkSamples) == g)
          samples[(size_t)row * kTopkSamples + i] = sc;
      }
    }
  }
}

// The multi-query form (4 query heads x 128 dims sharing one key head per
// group, 512 B of k̂ per group: OrcaRouter article on PR #41855, "Warum QSA
// der heikle Teil ist - in Zahlen"):
//   score[g] = sum_h w[h] * max(0, sum_d q[h,d] * khat[g,d])
// One wavefront consumes one 8 KiB page (16 groups): load i of lane l is
// float4 (l % 32) of group 2i + l / 32, so each half-wave holds one group's
// 128 dims and every lane keeps the matching 4 dims of all 4 query heads.
// A head's dot product finishes with a DPP row sum and one cross-row
// shuffle within the half-wave.
constexpr int kMqaHeads = 4, kMqaDim = 128;

__global__ __launch_bounds__(kScoreThreads) void index_score_gemv_mqa_kernel(
    const float* __restrict__ khat, const int32_t* __restrict__ page_table, int max_pages,
    int num_pages, const int32_t* __restrict__ row_req, const int32_t* __restrict__ row_len,
    int req0, int first_pos, int max_ctx, const float* __restrict__ q_idx,
    const float* __restrict__ w_idx, float* __restrict__ scores, int gstride,
    float* __restrict__ samples) {
  constexpr int kPageF4 = kGroupsPerPage * kMqaDim / 4;  // 512 float4 per page
  const int row = blockIdx.y;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int L = row_len ? row_len[row] : first_pos + row + 1;
  const int G = (L >= 0 && L <= max_ctx) ? L / kRatio : 0;
  const int req = row_req ? row_req[row] : (row_len ? row : req0);

  const int d0 = 4 * (lane & 31);
  const float* qrow = q_idx + (size_t)row * kMqaHeads * kMqaDim;
  float4 qh[kMqaHeads];
  float wh[kMqaHeads];
#pragma unroll
  for (int h = 0; h < kMqaHeads; ++h) {
    qh[h] = *reinterpret_cast<const float4*>(qrow + h * kMqaDim + d0);
    wh[h] = w_idx[(size_t)row * kMqaHeads + h];
  }

  float* srow = scores + (size_t)row * gstride;
  const int row_pages = (gstride + kGroupsPerPage - 1) / kGroupsPerPage;
  const int* pt = page_table + (size_t)req * max_pages;

  for (int i = 0; i < kPagesPerWave; ++i) {
    const int page = blockIdx.x * kScoreWaves * kPagesPerWave + i * kScoreWaves + wave;
    if (page >= row_pages) break;
    const int g0 = page * kGroupsPerPage;
    float sc = -INFINITY;
    if (g0 < G) {
      const int phys = pt[page];
      if (phys >= 0 && phys < num_pages) {
        const float4* base = reinterpret_cast<const float4*>(khat) + (size_t)phys * kPageF4;
        float v[kGroupsPerPage / 2];  // group 2j + lane / 32
#pragma unroll
        for (int j = 0; j < kGroupsPerPage / 2; ++j) {
          const float4 x = stream_load(base + j * kWave + lane);
          float s = 0.0f;
#pragma unroll
          for (int h = 0; h < kMqaHeads; ++h) {
            float p = row16_sum(dot4(x, qh[h]));
            p += __shfl_xor(p, 16, kWave);
            s += wh[h] * fmaxf(p, 0.0f);
          }
          v[j] = s;
        }
        // lane l < 16 takes group l from a lane of half l % 2 whose v index
        // is l / 2
        float mine = v[0];
#pragma unroll
        for (int j = 1; j < kGroupsPerPage / 2; ++j) mine = (((lane & 15) >> 1) == j) ? v[j] : mine;
        const float keep = __shfl(mine, (lane & 1) * 32 + (lane & 15), kWave);
        if (g0 + (lane & 15) < G) sc = keep + 0.0f;  // -0 -> +0
      }
    }
    if (lane < kGroupsPerPage && g0 + lane < gstride) {
      srow[g0 + lane] = sc;
      const int g = g0 + lane;
      if (samples && G >= kTopkSamples && g < G) {
        const int i = (int)(((long long)g * kTopkSamples + G - 1) / G);
        if (i < kTopkSamples && (int)(((long long)i * G) / kTopkSamples) == g)
          samples[(size_t)row * kTopkSamples + i] = sc;
      }
    }
  }
}

}  // namespace

hipError_t launch_index_score_gemv(const float* khat, const int32_t* page_table, int max_pages,
                                   int num_pages, int n_rows, const int32_t* row_req,
                                   const int32_t* row_len, int req0, int first_pos, int max_ctx,
                                   const float* q_idx, const float* w_idx, float* scores,
                                   int gstride, hipStream_t stream, float* samples,
                                   bool shared_key) {
  if (n_rows <= 0 || gstride <= 0) return hipSuccess;
  const int row_pages = (gstride + kGroupsPerPage - 1) / kGroupsPerPage;
  const int per_block = kScoreWaves * kPagesPerWave;
  dim3 grid((row_pages + per_block - 1) / per_block, n_rows, 1);
  auto kern = shared_key ? index_score_gemv_mqa_kernel : index_score_gemv_kernel;
  hipLaunchKernelGGL(kern, grid, dim3(kScoreThreads), 0, stream, khat,
                     page_table, max_pages, num_pages, row_req, row_len, req0, first_pos, max_ctx,
                     q_idx, w_idx, scores, gstride, samples);
  return hipGetLastError();
}

}  // namespace qsa
