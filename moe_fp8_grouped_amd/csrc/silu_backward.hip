// moe_silu_mul_backward: gradients of the gated FFN's activation
// h = silu(a) * b for an upstream gradient dh, the activation step of the
// layer backward that "Support quantization for tokamax gmm v2" splits into
// gmm / tgmm calls ("What this does").  The pages do not discuss the
// activation; the recipe is pinned in float32, one rounding per step, no
// fused multiply-add, so the result is defined to the bit:
//   den = 1 + e(-a)        (the pinned exp of the forward, common.hpp)
//   s   = 1 / den,  q = a / den               (IEEE divides)
//   db  = dh * q
//   da  = (dh * b) * (s * (1 + a * (1 - s)))
// then each rounded to bfloat16 (nearest even).  Elementwise and HBM-bound:
// 6 bytes read and 4 written per element.  a and b may be the column halves
// of one [R, 2C] buffer (row stride lda), and da / db the halves of another
// (row stride ldo), the layout the input-gradient grouped matmul over
// [W0 | W1]^T reads.
#include "common.hpp"

namespace moe {
namespace {

// The two quotients 1 / den and a / den by the forward's reciprocal-and-
// correction sequence (silu_quotient, correctly rounded for these operands --
// the GPU test over every finite bfloat16 gate compares both results bit for
// bit with IEEE division), the IEEE divide when den exceeds 2^126.
__device__ __forceinline__ void silu_bwd1(float a, float b, float dh, float& da, float& db) {
#pragma clang fp contract(off)
  const float den = 1.0f + pinned_exp(-a);
  float s, q;
  if (den <= 0x1p126f) {
    s = silu_quotient(1.0f, den);
    q = silu_quotient(a, den);
  } else {
    s = 1.0f / den;
    q = a / den;
  }
  db = dh * q;
  const float ds = s * (1.0f + a * (1.0f - s));
  da = (dh * b) * ds;
}

__device__ __forceinline__ float lo16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// One thread per 8-element chunk (grid-stride).
__global__ __launch_bounds__(256) void silu_mul_bwd_kernel(const uint16_t* __restrict__ a,
                                                           const uint16_t* __restrict__ b, int64_t lda,
                                                           const uint16_t* __restrict__ dh, int64_t R, int64_t C,
                                                           uint16_t* da, uint16_t* db, int64_t ldo) {
  const int64_t cpr = C >> 3;
  const int64_t total = R * cpr;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t r = i / cpr, c = (i - r * cpr) * 8;
    const uint4 av = *reinterpret_cast<const uint4*>(a + r * lda + c);
    const uint4 bv = *reinterpret_cast<const uint4*>(b + r * lda + c);
    const uint4 dv = *reinterpret_cast<const uint4*>(dh + r * C + c);
    const uint32_t aw[4] = {av.x, av.y, av.z, av.w}, bw[4] = {bv.x, bv.y, bv.z, bv.w},
                   dw[4] = {dv.x, dv.y, dv.z, dv.w};
    uint32_t oa[4], ob[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float a0, b0, a1, b1;
      silu_bwd1(lo16(aw[k]), lo16(bw[k]), lo16(dw[k]), a0, b0);
      silu_bwd1(hi16(aw[k]), hi16(bw[k]), hi16(dw[k]), a1, b1);
      oa[k] = f32_to_bf16(a0) | (static_cast<uint32_t>(f32_to_bf16(a1)) << 16);
      ob[k] = f32_to_bf16(b0) | (static_cast<uint32_t>(f32_to_bf16(b1)) << 16);
    }
    *reinterpret_cast<uint4*>(da + r * ldo + c) = make_uint4(oa[0], oa[1], oa[2], oa[3]);
    *reinterpret_cast<uint4*>(db + r * ldo + c) = make_uint4(ob[0], ob[1], ob[2], ob[3]);
  }
}

}  // namespace
}  // namespace moe

extern "C" int moe_silu_mul_backward(const void* a, const void* b, int64_t lda, const void* dh, int64_t R,
                                     int64_t C, void* da, void* db, int64_t ldo, void* stream) {
  if (R < 0 || C <= 0 || C % 8 || lda < C || lda % 8 || ldo < C || ldo % 8) return MOE_ERR_SHAPE;
  if (R == 0) return MOE_OK;
  if (!a || !b || !dh || !da || !db) return MOE_ERR_NULL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t chunks = R * (C / 8);
  int64_t blocks = moe_cdiv(chunks, 256);
  if (blocks > 16384) blocks = 16384;
  moe::silu_mul_bwd_kernel<<<static_cast<unsigned>(blocks), 256, 0, st>>>(
      static_cast<const uint16_t*>(a), static_cast<const uint16_t*>(b), lda, static_cast<const uint16_t*>(dh), R, C,
      static_cast<uint16_t*>(da), static_cast<uint16_t*>(db), ldo);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}
