// Decoded rows of one cache row, for checking (rotated basis, fp32).
//
// Window rows are bf16 widened to fp32; an INT2 row is scale * code + zero
// (OScaR notes, "integer quantization basics": x_hat = Delta (Q - z), with the
// zero point stored as the fp16 value of the group's lower clip limit).
// scale * code is exact in fp32 (11-bit times 2-bit), so the fused
// multiply-add rounds the exact value once.  In OScaR key mode an INT2 key is
// s * (Delta * (code - z)) in fp64 (OScaR notes, step two "Omni-Token
// Scaling"), or s * z for a constant channel, rounded once to fp32; the
// channel's (Delta, z) sit in the page of its half of the key block.
#include "device_common.h"

namespace oscar {

__global__ __launch_bounds__(128) void dequant_kernel(CacheArgs c, int slot, int len, int t0,
                                                      float* __restrict__ k_out,
                                                      float* __restrict__ v_out) {
  const int p = t0 + blockIdx.x, h = blockIdx.y, ch = threadIdx.x;
  const int sq = s_quant_of(len, c.s_sink, c.s_keep, c.s_flush);
  const size_t o = ((size_t)blockIdx.x * c.hkv + h) * kD + ch;
  float kv, vv;
  if (p < c.s_sink || p >= sq) {
    int blk, tt;
    if (p < c.s_sink) {
      blk = p / kPage;
      tt = p % kPage;
    } else {
      const int r = (p - c.s_sink) % c.ring_cap;
      blk = c.sink_blocks + r / kPage;
      tt = r % kPage;
    }
    const uint16_t* wb =
        c.win + (((size_t)slot * c.hkv + h) * c.win_blocks + blk) * (2 * kPage * kD);
    kv = bf16_bits_to_f32(wb[tt * kD + ch]);
    vv = bf16_bits_to_f32(wb[kPage * kD + 32 * (16 * (tt >> 2) + (ch >> 3)) + 4 * (ch & 7) +
                             (tt & 3)]);
  } else {
    const int m = (p - c.s_sink) / kPage, t = (p - c.s_sink) % kPage;
    const int phys = m < c.max_pages ? c.block_table[(size_t)slot * c.max_pages + m] : -1;
    if (phys < 0 || phys >= c.num_pages) {
      kv = vv = __builtin_nanf("");
    } else {
      const uint8_t* base = c.pages + ((size_t)phys * c.hkv + h) * c.page_bytes;
      const uint32_t* kw = (const uint32_t*)base;
      const uint32_t* vw = (const uint32_t*)(base + 512);
      const uint32_t* kp = (const uint32_t*)(base + 1024);
      const uint32_t* vp = (const uint32_t*)(base + v_param_offset(c));
      const uint32_t kc = (kw[8 * t + ch / 16] >> (2 * (ch % 16))) & 3u;
      const uint32_t vc =
          (vw[2 * (16 * (t >> 2) + ch / 8) + ((t & 3) >> 1)] >> (16 * (t & 1) + 2 * (ch % 8))) & 3u;
      const int gr = ch / c.group;
      const uint32_t kpw = kp[16 * gr + t], vpw = vp[16 * gr + t];
      const float ks = (float)__builtin_bit_cast(_Float16, (uint16_t)(kpw & 0xFFFFu));
      const float kz = (float)__builtin_bit_cast(_Float16, (uint16_t)(kpw >> 16));
      const float vs = (float)__builtin_bit_cast(_Float16, (uint16_t)(vpw & 0xFFFFu));
      const float vz = (float)__builtin_bit_cast(_Float16, (uint16_t)(vpw >> 16));
      kv = __builtin_fmaf(ks, (float)kc, kz);
      vv = __builtin_fmaf(vs, (float)vc, vz);
      if (c.key_mode) {
        const int mc = (m & ~1) + (ch >> 6);   // page holding channel ch's (Delta, z)
        const int pc = mc < c.max_pages ? c.block_table[(size_t)slot * c.max_pages + mc] : -1;
        if (pc < 0 || pc >= c.num_pages) {
          kv = __builtin_nanf("");
        } else {
          const uint8_t* cb = c.pages + ((size_t)pc * c.hkv + h) * c.page_bytes;
          const uint32_t cw = ((const uint32_t*)(cb + kOtsChanOffset))[ch & 63];
          const double dl = (double)bf16_bits_to_f32(cw & 0xFFFFu);
          const double z = (double)bf16_bits_to_f32(cw >> 16);
          const double sv =
              (double)bf16_bits_to_f32(((const uint16_t*)(base + kOtsScaleOffset))[t]);
          const double un = dl == 0.0 ? z : dl * ((double)kc - z);
          kv = (float)(sv * un);
        }
      }
    }
  }
  k_out[o] = kv;
  v_out[o] = vv;
}

hipError_t launch_dequant(const CacheArgs& c, int slot, int len, int t0, int t1, float* k_out,
                          float* v_out, hipStream_t stream) {
  if (t1 <= t0) return hipSuccess;
  dim3 grid(t1 - t0, c.hkv);
  hipLaunchKernelGGL(dequant_kernel, grid, dim3(128), 0, stream, c, slot, len, t0, k_out, v_out);
  return hipGetLastError();
}

}  // namespace oscar
