// Nested KV4 / KV8 cache ("BitNest: Bit-Nested Speculative Decoding for
// Memory-Efficient LLM Inference Acceleration", Sec. 3.4 and Sec. A.2):
// quantization on write, the quantizing commit, and the dequantization helpers
// of the verify attention over the code planes (attn_nested_lds.hpp).
//
// Format (per token and KV head, D elements):
//   s = max|x| / 7, t = x / s, q4 = rint(t), qr = clamp(rint(16 t) - 16 q4, -8, 7)
//   (fp32, round half to even); KV4 = s q4, KV8 = (s / 16)(16 q4 + qr).
//   Codes are stored + 8 as nibbles, two per byte, even element low:
//   base / ref planes [pages, Hkv, 16, D/2] bytes, scales [pages, Hkv, 16] fp32.
//
// Codes as MFMA operands: with both nibbles of an element, the byte
// u = 16 (q4 + 8) + (qr + 8) = c8 + 136, c8 = 16 q4 + qr, is built for four
// elements at a time with two masks and a shift, and enters the bf16 MFMA as
// the bit pattern 0x00uu, which is exactly u 2^-133 (attn_nested_lds.hpp).
// The products therefore see u instead of c8; the offset is removed in fp32:
//   scores: q.k = (s_k / 16) (sum_d q_d u_d - 136 sum_d q_d) per key,
//   values: sum_t p_t v_t = (sum_t p_t s_t u_t - 136 sum_t p_t s_t) / 16,
// with sum_d q_d computed once per row and sum_t p_t s_t kept beside the row
// sum.  A KV4 read uses the refinement nibble 8 (qr = 0).
#pragma once

#include "accept_commit.hpp"
#include "common.hpp"

namespace mtpv {

constexpr float kNestByteOffset = 136.f;   // u = c8 + 136
constexpr unsigned kNestZeroRef = 0x88888888u;  // eight refinement codes 0

// ---------------------------------------------------------------------------
// quantization
// ---------------------------------------------------------------------------

__device__ __forceinline__ float load_elem(const void* p, int dtype, size_t i) {
  if (dtype == MTP_F32) return static_cast<const float*>(p)[i];
  return bf16_bits_to_float(static_cast<const unsigned short*>(p)[i]);
}

// Quantizes one vector of D <= 128 elements by one wave: lane l takes
// elements 2l and 2l + 1 and writes byte l of both planes; lane 0 writes the
// scale.  All lanes of the wave must be active.
__device__ __forceinline__ void wave_quantize(const void* x, int dtype, int D, uint8_t* base,
                                              uint8_t* ref, float* scale) {
  const int lane = threadIdx.x & 63;
  const bool in = 2 * lane < D;
  const float x0 = in ? load_elem(x, dtype, 2 * lane) : 0.f;
  const float x1 = in ? load_elem(x, dtype, 2 * lane + 1) : 0.f;
  const float amax = wave_max(fmaxf(fabsf(x0), fabsf(x1)));
  const float s = amax / 7.f;  // IEEE division, as the definition states
  const bool live = s > 0.f;
  const float t0 = live ? x0 / s : 0.f;
  const float t1 = live ? x1 / s : 0.f;
  const float a0 = rintf(t0), a1 = rintf(t1);
  const float r0 = fminf(fmaxf(rintf(16.f * t0) - 16.f * a0, -8.f), 7.f);
  const float r1 = fminf(fmaxf(rintf(16.f * t1) - 16.f * a1, -8.f), 7.f);
  if (in) {
    base[lane] = (uint8_t)(((int)a0 + 8) | (((int)a1 + 8) << 4));
    ref[lane] = (uint8_t)(((int)r0 + 8) | (((int)r1 + 8) << 4));
  }
  if (lane == 0) *scale = s;
}

// Row index of slot (page, head, slot) in the planes (rows of D/2 bytes, or one scale).
__device__ __forceinline__ size_t nest_row(int page, int h, int slot, int Hkv) {
  return ((size_t)page * Hkv + h) * kPage + slot;
}

struct QuantizeParams {
  const void* k_rows;  // [n, Hkv, D]
  const void* v_rows;
  const int32_t* slots;  // [n]: page * 16 + slot
  mtp_nested_kv kv;
  int n, Hkv, D, dtype, num_pages;
};

// One wave per (row, KV head, K or V).
__global__ __launch_bounds__(256) void kv_quantize_kernel(QuantizeParams p) {
  const long item = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= (long)p.n * p.Hkv * 2) return;
  const bool is_v = item & 1;
  const int h = (int)((item >> 1) % p.Hkv);
  const int r = (int)((item >> 1) / p.Hkv);
  const int slot = p.slots[r];
  if (slot < 0 || slot >= p.num_pages * kPage) {
    if ((threadIdx.x & 63) == 0) raise_status(MTP_DEV_BAD_PAGE);
    return;
  }
  const size_t row = nest_row(slot >> 4, h, slot & 15, p.Hkv);
  const size_t src = ((size_t)r * p.Hkv + h) * p.D;
  const int esz = p.dtype == MTP_F32 ? 4 : 2;
  const char* x = static_cast<const char*>(is_v ? p.v_rows : p.k_rows) + src * esz;
  if (is_v)
    wave_quantize(x, p.dtype, p.D, p.kv.v_base + row * (p.D / 2), p.kv.v_ref + row * (p.D / 2),
                  p.kv.v_scale + row);
  else
    wave_quantize(x, p.dtype, p.D, p.kv.k_base + row * (p.D / 2), p.kv.k_ref + row * (p.D / 2),
                  p.kv.k_scale + row);
}

struct NestedCommitParams {
  CommitParams c;  // k_cache / v_cache / row_bytes unused
  mtp_nested_kv kv;
  int Hkv, D, dtype;
};

// The commit of the accepted rows into a nested cache: the plan of the plain
// commit, then each accepted (position, KV head, K or V) vector is quantized
// by one wave into its slot.
__global__ __launch_bounds__(256) void commit_nested_kernel(NestedCommitParams p) {
  __shared__ int s_src[MTP_MAX_W];
  __shared__ int s_dst[MTP_MAX_W];
  __shared__ int s_meta[2];
  const int b = blockIdx.x;
  commit_plan<false>(p.c, b, commit_prefetch(p.c, b), 0, nullptr, s_src, s_dst, s_meta);
  const int a = s_meta[0];
  const int first = s_meta[1];
  if (a < first) return;
  const int per = p.Hkv * 2;
  const int total = (a - first + 1) * per;
  const int esz = p.dtype == MTP_F32 ? 4 : 2;
  for (int item = threadIdx.x >> 6; item < total; item += blockDim.x >> 6) {
    const int k = first + item / per;
    const int h = (item % per) >> 1;
    const bool is_v = item & 1;
    const int dst = s_dst[k];
    const size_t row = nest_row(dst >> 4, h, dst & 15, p.Hkv);
    const size_t src = (((size_t)b * p.c.W + s_src[k]) * p.Hkv + h) * p.D;
    const char* x = static_cast<const char*>(is_v ? p.c.v_new : p.c.k_new) + src * esz;
    if (is_v)
      wave_quantize(x, p.dtype, p.D, p.kv.v_base + row * (p.D / 2), p.kv.v_ref + row * (p.D / 2),
                    p.kv.v_scale + row);
    else
      wave_quantize(x, p.dtype, p.D, p.kv.k_base + row * (p.D / 2), p.kv.k_ref + row * (p.D / 2),
                    p.kv.k_scale + row);
  }
}

// ---------------------------------------------------------------------------
// dequantization into MFMA operands
// ---------------------------------------------------------------------------

// Bytes u = c8 + 136 of 8 elements from their base and refinement dwords:
// `ev` holds elements 0, 2, 4, 6 (byte k = element 2k), `od` elements 1, 3, 5, 7.
__device__ __forceinline__ void nest_bytes(unsigned b, unsigned r, unsigned& ev, unsigned& od) {
  ev = ((b & 0x0F0F0F0Fu) << 4) | (r & 0x0F0F0F0Fu);
  od = (b & 0xF0F0F0F0u) | ((r >> 4) & 0x0F0F0F0Fu);
}

struct NestedAttn {
  mtp_nested_kv kv;
  int kv8_recent;  // -1: all KV8; 0: all KV4; N: the N newest committed tokens in KV8
};

}  // namespace mtpv
