// append.hip — cache append: the keys and values of new tokens are written
// into the paged KV cache in its element format, and the compressed indexer
// keys of the groups those tokens complete into the paged k̂ cache.
//
// The qsa-hisparse README lists "prefill writes" among the attention
// backend's duties and fixes FP8 E4M3 KV with page size 64 in its offload
// contract; it prints no quantiser.  This library's reading: a stored
// element is the binary32 quotient x / scale of the new bf16 value x and the
// cache's per-tensor scale (the factor attention decodes with), rounded to
// the nearest FP8 E4M3FN code (ties to an even mantissa; magnitudes above
// 448 saturate to 448), or to the nearest bfloat16 for a BF16 cache.
//
// Both kernels are plain streaming copies (HBM-bound): a thread moves 16
// bytes of one token's [Hkv, D] row of K and of V, or 16 bytes of one k̂
// group, so a wavefront covers 1 KiB of contiguous input and output.
#include "qsa_device.h"
#include "qsa_launch.h"

namespace qsa {
namespace {

// Nearest E4M3FN code of a binary32 value (see the file comment).  Normal
// range: the fp32 exponent is re-biased (127 -> 7) and the 23-bit mantissa
// rounded to 3 bits, nearest-even, a carry moving into the exponent.  Below
// 2^-6 the code is the nearest multiple of 2^-9 (the subnormal step), which
// reaches 8 = the smallest normal exactly when it should.
__device__ __forceinline__ uint32_t fp8_e4m3_code(float q) {
  const uint32_t sign = (__float_as_uint(q) >> 24) & 0x80u;
  const float a = fabsf(q);
  if (!(a == a)) return 0x7Fu;
  if (a >= 448.0f) return sign | 0x7Eu;
  if (a < 0x1p-6f) return sign | (uint32_t)__builtin_rintf(a * 512.0f);
  uint32_t b = __float_as_uint(a);
  b += 0x7FFFFu + ((b >> 20) & 1u);
  return sign | ((b >> 20) - (120u << 3));
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  if (!(x == x)) return (u >> 16) | 0x40u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

struct AppendArgs {
  void* k_cache;
  void* v_cache;
  float* khat_cache;
  const int32_t* page_table;
  int max_pages, num_pages;
  int n_req, n_tokens;
  const int32_t* req_rows;
  const int32_t* start_pos;
  const uint16_t* k_new;
  const uint16_t* v_new;
  const float* khat_new;
  int khat_slots;
  int group_f4;   // float4 per k̂ group: 128 (8 heads x 64) or 32 (one key of 128)
  int row_elems;  // Hkv * D
  float k_scale, v_scale;
};

// 8 new bf16 values -> their stored form, 8 bytes (FP8) or 16 bytes (BF16)
template <bool kFp8>
__device__ __forceinline__ void store8(void* cache, long long dst, qsa_u4v x, float scale) {
  if constexpr (kFp8) {
    uint32_t w[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t packed = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t half = (j & 1) ? (x[2 * h + j / 2] >> 16) : (x[2 * h + j / 2] & 0xFFFFu);
        packed |= fp8_e4m3_code(bf16_to_f32(half) / scale) << (8 * j);
      }
      w[h] = packed;
    }
    *reinterpret_cast<uint2*>(static_cast<uint8_t*>(cache) + dst) = make_uint2(w[0], w[1]);
  } else {
    qsa_u4v y = x;
    if (scale != 1.0f) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t lo = f32_to_bf16_rne(bf16_to_f32(x[k] & 0xFFFFu) / scale);
        const uint32_t hi = f32_to_bf16_rne(bf16_to_f32(x[k] >> 16) / scale);
        y[k] = lo | (hi << 16);
      }
    }
    *reinterpret_cast<qsa_u4v*>(static_cast<uint16_t*>(cache) + dst) = y;
  }
}

__device__ __forceinline__ void append_khat(const AppendArgs& a, long long idx);

// One launch does both parts: the first kv_blocks workgroups move K/V, the
// rest the k̂ of completed groups.
template <bool kFp8>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a, int kv_blocks) {
  if ((int)blockIdx.x >= kv_blocks) {
    append_khat(a, (long long)(blockIdx.x - kv_blocks) * blockDim.x + threadIdx.x);
    return;
  }
  const int chunks = a.row_elems / 8;  // 16-byte pieces of a token's row
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long long)a.n_req * a.n_tokens * chunks) return;
  const long long tok = idx / chunks;  // request r, new token i
  const int c = (int)(idx - tok * chunks);
  const int r = (int)(tok / a.n_tokens), i = (int)(tok - (long long)r * a.n_tokens);
  // the new values first: their address does not depend on the page, so
  // they are in flight while the position and the page id are looked up
  const long long src = tok * a.row_elems + 8 * c;
  const qsa_u4v kx = stream_load_u4(a.k_new + src);
  const qsa_u4v vx = stream_load_u4(a.v_new + src);
  const long long t = (long long)a.start_pos[r] + i;
  if (t < 0 || t / kPage >= a.max_pages) return;
  const int32_t p = a.page_table[(long long)a.req_rows[r] * a.max_pages + t / kPage];
  if (p < 0 || p >= a.num_pages) return;
  const long long dst = ((long long)p * kPage + t % kPage) * a.row_elems + 8 * c;
  store8<kFp8>(a.k_cache, dst, kx, a.k_scale);
  store8<kFp8>(a.v_cache, dst, vx, a.v_scale);
}

__device__ __forceinline__ void append_khat(const AppendArgs& a, long long idx) {
  const int kF4 = a.group_f4;
  if (!a.khat_new || idx >= (long long)a.n_req * a.khat_slots * kF4) return;
  const long long slot = idx / kF4;  // request r, slot j
  const int f = (int)(idx - slot * kF4);
  const int r = (int)(slot / a.khat_slots), j = (int)(slot - (long long)r * a.khat_slots);
  // the new k̂ first (its address does not depend on the page)
  const float4 v = stream_load(reinterpret_cast<const float4*>(a.khat_new) + slot * kF4 + f);
  const long long s0 = a.start_pos[r];
  const long long g0 = s0 >= 0 ? s0 / kRatio : -((-s0 + kRatio - 1) / kRatio);  // floor
  const long long g = g0 + j, last = g * kRatio + kRatio - 1;
  if (g < 0 || last < s0 || last >= s0 + a.n_tokens) return;
  if (g / kGroupsPerPage >= a.max_pages) return;
  const int32_t p = a.page_table[(long long)a.req_rows[r] * a.max_pages + g / kGroupsPerPage];
  if (p < 0 || p >= a.num_pages) return;
  reinterpret_cast<float4*>(a.khat_cache)[((long long)p * kGroupsPerPage + g % kGroupsPerPage) *
                                              kF4 + f] = v;
}

}  // namespace

hipError_t launch_append(void* k_cache, void* v_cache, float* khat_cache,
                         const int32_t* page_table, int max_pages, int num_pages, int n_req,
                         const int32_t* req_rows, const int32_t* start_pos, int n_tokens,
                         const uint16_t* k_new, const uint16_t* v_new, const float* khat_new,
                         int khat_group_floats, int row_elems, int kv_dtype, float k_scale,
                         float v_scale, hipStream_t stream) {
  if (n_req <= 0 || n_tokens <= 0) return hipSuccess;
  AppendArgs a{k_cache, v_cache, khat_cache, page_table, max_pages, num_pages, n_req, n_tokens,
               req_rows, start_pos, k_new, v_new, khat_new, (n_tokens + kRatio - 1) / kRatio,
               khat_group_floats / 4, row_elems, k_scale, v_scale};
  const long long n_kv = (long long)n_req * n_tokens * (row_elems / 8);
  const int blocks_kv = (int)((n_kv + 255) / 256);
  const long long n_kh = khat_new ? (long long)n_req * a.khat_slots * a.group_f4 : 0;
  const int blocks = blocks_kv + (int)((n_kh + 255) / 256);
  auto kern = kv_dtype == 1 ? append_kernel<true> : append_kernel<false>;
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(256), 0, stream, a, blocks_kv);
  return hipGetLastError();
}

}  // namespace qsa
