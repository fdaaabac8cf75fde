// Decode-step preparation on gfx950: new index vectors get RoPE and their storage
// type, new latent rows are appended to the latent cache.
//
// RoPE follows the Megatron-Bridge GLM-5 DSA pull request (commit on the indexer
// RoPE half swap): the LAST D/2 dims of every index head are rotated, rotate-half
// pairs (i, i + D/4) turning by pos * theta^(-2i/(D/2)) (rope_theta = 8e6 in the
// same pull request's config fix).  The angle is formed in double precision (for
// positions up to 2^20 a float32 angle would be off by whole hundredths of a
// radian); the rotated vector is rounded to float32, then stored as bf16 (round to
// nearest even) or as fp8 e4m3fn with one float32 scale per (token, head):
// scale = amax / 448 (1 if amax is 0), code = e4m3fn(y / scale) rounded to nearest
// even and saturated at 448.  Both divisions are IEEE round-to-nearest.
#include "dsa_internal.h"

namespace dsa {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));

// float32 -> OCP e4m3fn code (1 sign, 4 exponent bits with bias 7, 3 mantissa bits;
// exponent field 0 holds m * 2^-9): round to nearest even, magnitudes at or above 448
// saturate to 448 (code 0x7E).  NaN inputs give an unspecified code.
__device__ __forceinline__ uint8_t e4m3_from_f32(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = fabsf(x);
  if (!(a < 448.f)) return (uint8_t)(sign | 0x7Eu);
  if (a < 0.015625f) {  // below 2^-6: multiples of 2^-9 (8 * 2^-9 is the smallest normal, code 8)
    return (uint8_t)(sign | (uint32_t)__builtin_rintf(a * 512.f));
  }
  int e = (int)((u >> 23) & 0xFFu) - 127;           // -6 .. 8
  uint32_t sig = (u & 0x7FFFFFu) | 0x800000u;      // 24-bit significand
  uint32_t q = sig >> 20;                           // 8 .. 15: implicit bit + 3 mantissa bits
  const uint32_t rem = sig & 0xFFFFFu, halfway = 0x80000u;
  if (rem > halfway || (rem == halfway && (q & 1u))) ++q;
  if (q == 16u) {
    q = 8u;
    ++e;
  }
  uint32_t code = ((uint32_t)(e + 7) << 3) | (q - 8u);
  if (code > 0x7Eu) code = 0x7Eu;
  return (uint8_t)(sign | code);
}

__device__ __forceinline__ uint16_t bf16_from_f32(float x) {
  const uint32_t u = __float_as_uint(x);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// One 64-thread workgroup per vector (token n, head h).
__global__ __launch_bounds__(64) void index_prep_kernel(PrepParams p) {
  __shared__ float y[1024];
  const int lane = threadIdx.x;
  const int64_t v = blockIdx.x;
  const int64_t n = v / p.heads;
  const int h = (int)(v % p.heads);
  const int64_t row = p.rows ? p.rows[n] : n;
  if (row < 0 || row >= p.n_rows) return;  // the whole workgroup leaves together
  const int D = p.D, r = D / 2, half = r / 2, front = D - r;
  const float* x = p.x + v * D;
  for (int j = lane; j < front; j += 64) y[j] = x[j];
  const double pos = (double)p.pos[n];
  for (int i = lane; i < half; i += 64) {
    const double inv = pow((double)p.theta, -2.0 * (double)i / (double)r);
    double s, c;
    sincos(pos * inv, &s, &c);
    const double a = x[front + i], b = x[front + half + i];
    y[front + i] = (float)(a * c - b * s);
    y[front + half + i] = (float)(b * c + a * s);
  }
  __syncthreads();
  const int64_t o = (row * p.heads + h) * (int64_t)D;
  if (p.out_dtype == BF16) {
    uint16_t* out = static_cast<uint16_t*>(p.out) + o;
    for (int j = lane; j < D; j += 64) out[j] = bf16_from_f32(y[j]);
    return;
  }
  float amax = 0.f;
  for (int j = lane; j < D; j += 64) amax = fmaxf(amax, fabsf(y[j]));
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  const float scale = amax > 0.f ? __fdiv_rn(amax, 448.f) : 1.f;
  uint8_t* out = static_cast<uint8_t*>(p.out) + o;
  for (int j = lane; j < D; j += 64) out[j] = e4m3_from_f32(__fdiv_rn(y[j], scale));
  if (lane == 0) p.out_scale[row * p.heads + h] = scale;
}

// One 64-thread workgroup per new token: its latent row (row_bytes, a multiple of 16)
// is copied to its cache row.
__global__ __launch_bounds__(64) void latent_append_kernel(LatentAppendParams p) {
  const int64_t n = blockIdx.x;
  const int64_t row = p.rows[n];
  if (row < 0 || row >= p.n_rows) return;
  const int chunks = p.row_bytes / 16;
  const i32x4* src = reinterpret_cast<const i32x4*>(static_cast<const unsigned char*>(p.src) + n * p.row_bytes);
  i32x4* dst = reinterpret_cast<i32x4*>(static_cast<unsigned char*>(p.dst) + row * p.row_bytes);
  for (int c = threadIdx.x; c < chunks; c += 64) dst[c] = src[c];
}

}  // namespace

hipError_t launch_index_prep(const PrepParams& p, hipStream_t st) {
  const int64_t vecs = (int64_t)p.n * p.heads;
  if (vecs == 0) return hipSuccess;
  hipLaunchKernelGGL(index_prep_kernel, dim3((unsigned)vecs), dim3(64), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_latent_append(const LatentAppendParams& p, hipStream_t st) {
  if (p.n == 0) return hipSuccess;
  hipLaunchKernelGGL(latent_append_kernel, dim3((unsigned)p.n), dim3(64), 0, st, p);
  return hipGetLastError();
}

}  // namespace dsa
