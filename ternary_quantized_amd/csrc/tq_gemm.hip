// Prefill GEMM over row-split ternary planes:
//   Y[m][n] = sum_g s[n][g] * sum_{j in g} t[n][j] * X[m][j]
// [ninfer-skill] §3 (planes), [gguf-explainer] §4.3 (codes), [tensorsharp]
// §4.4 (every low-bit projection multiplies the rotated activations).
//
// This is a genuinely dense contraction, so it runs on the matrix cores
// (v_mfma_f32_32x32x16_f16, fp32 accumulation).  Each K step is one
// 128-weight group: the workgroup stages its X tile in LDS as binary16 and
// decodes its weight tile into LDS as the binary16 values t*s.  That value is
// exact -- s is itself a binary16 and t is -1, 0 or +1 -- so folding the
// group scale into the decoded weight loses nothing, and the only rounding
// before the fp32 accumulation is that of X to binary16.
//
// Workgroup: 256 threads (4 waves in a 2x2 arrangement), a 128x128 output
// tile, each wave a 64x64 sub-tile of 2x2 MFMA blocks of 32x32.
// Workgroups are numbered N-tile-major inside each M-tile band and the band
// is chosen from the XCD the workgroup lands on (workgroups are dealt to the
// 8 XCDs round-robin), so the workgroups that share an X tile share an L2.

#include "tq_device.h"
#include "tq_launch.h"

namespace tq {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int GM = 128, GN = 128, GK = 128;
constexpr int LDSROW = GK + 8;  // halves per LDS row (16-byte pad)

__device__ __forceinline__ half2_t cvt_pair(uint32_t v, int sel) {
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, 1.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, 1.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, 1.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, 1.0f, 3);
  }
}

__device__ __forceinline__ uint32_t h2_bits(half2_t h) {
  uint32_t u;
  __builtin_memcpy(&u, &h, 4);
  return u;
}

// fp4 pair (u/2, v/2) -> (u-1)*s, (v-1)*s exactly: fma(c/2, 2s, -s).
__device__ __forceinline__ uint32_t scale_pair(half2_t c_half, half2_t s2, half2_t neg_s) {
  return h2_bits(__builtin_elementwise_fma(c_half, s2, neg_s));
}

// PQ2_0: one dword = 16 codes (weights 16d..16d+15, LSB pair first) ->
// 8 binary16 pairs in natural order, each value (code-1)*s.
__device__ __forceinline__ void decode_pq2_dword(uint32_t d, half2_t s2, half2_t ns,
                                                 uint32_t out[8]) {
  // byte q of p01 holds codes 4q (low nibble) and 4q+1 (high nibble);
  // byte q of p23 holds codes 4q+2 and 4q+3.
  const uint32_t p01 = (d & 0x03030303u) | ((d << 2) & 0x30303030u);
  const uint32_t p23 = ((d >> 4) & 0x03030303u) | ((d >> 2) & 0x30303030u);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    out[2 * q] = scale_pair(cvt_pair(p01, q), s2, ns);
    out[2 * q + 1] = scale_pair(cvt_pair(p23, q), s2, ns);
  }
}

// PTQ1_0: trits 5b..5b+4 of a base byte v (digit i = v/3^i mod 3).
__device__ __forceinline__ void ptq1_digits(uint32_t v, int n, uint32_t *d) {
  for (int i = 0; i < n; ++i) { d[i] = v % 3u; v /= 3u; }
}

template <int FMT, int XD, int YD>
__global__ __launch_bounds__(256) void gemm_kernel(Planes p, const uint16_t *__restrict__ X,
                                                   int64_t M, int64_t ldx, void *__restrict__ Y,
                                                   int64_t ldy, int tiles_n, int tiles_m) {
  __shared__ __attribute__((aligned(16))) _Float16 As[GM * LDSROW];
  __shared__ __attribute__((aligned(16))) _Float16 Bs[GN * LDSROW];

  // XCD-aware tile order: workgroup b runs on XCD b % 8; consecutive slots
  // on one XCD walk the N tiles of one M band.
  const int nwg = tiles_n * tiles_m;
  const int b = blockIdx.x;
  int tile;
  if (nwg % 8 == 0) {
    const int per_xcd = nwg / 8;
    tile = (b % 8) * per_xcd + b / 8;
  } else {
    tile = b;
  }
  const int tm = tile / tiles_n, tn = tile % tiles_n;
  const int64_t m0 = (int64_t)tm * GM, n0 = (int64_t)tn * GN;

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;

  floatx16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  for (int64_t g = 0; g < p.groups; ++g) {
    __syncthreads();
    // ---- stage X[m0:m0+128][128g:128g+128] as binary16
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int idx = t + 256 * i;
      const int r = idx >> 4, c8 = (idx & 15) * 8;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (m0 + r < M) {
        v = *reinterpret_cast<const uint4 *>(X + (m0 + r) * ldx + g * GK + c8);
        if constexpr (XD == DT_BF16) {
          uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t lo = f32_to_f16(bf16_to_f32((uint16_t)(w[e] & 0xFFFF)));
            const uint32_t hi = f32_to_f16(bf16_to_f32((uint16_t)(w[e] >> 16)));
            w[e] = lo | (hi << 16);
          }
          v = make_uint4(w[0], w[1], w[2], w[3]);
        }
      }
      *reinterpret_cast<uint4 *>(&As[r * LDSROW + c8]) = v;
    }
    // ---- decode W[n0:n0+128][group g] into t*s binary16
    if constexpr (FMT == FMT_PQ2) {
      const int r = t >> 1, half = t & 1;  // 64 weights per thread
      uint32_t o[32];
      if (n0 + r < p.n) {
        const int64_t row = n0 + r;
        const uint4 q = *reinterpret_cast<const uint4 *>(p.base + row * p.base_row + g * 32 +
                                                          16 * half);
        const _Float16 s = (_Float16)f16_to_f32(p.scale[row * p.groups + g]);
        half2_t s2, ns;
        s2.x = s2.y = (_Float16)(2.0f * (float)s);
        ns.x = ns.y = -s;
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int d = 0; d < 4; ++d) decode_pq2_dword(w[d], s2, ns, o + 8 * d);
      } else {
#pragma unroll
        for (int i = 0; i < 32; ++i) o[i] = 0;
      }
      uint4 *dst = reinterpret_cast<uint4 *>(&Bs[r * LDSROW + 64 * half]);
#pragma unroll
      for (int i = 0; i < 8; ++i) dst[i] = make_uint4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
    } else {
      // two quarter-groups (32 trits) per thread
#pragma unroll
      for (int rep = 0; rep < 2; ++rep) {
        const int qi = t + 256 * rep;  // 0..511
        const int r = qi >> 2, q = qi & 3;
        _Float16 vals[32];
        if (n0 + r < p.n) {
          const int64_t row = n0 + r;
          const uint8_t *bb = p.base + row * p.base_row + g * 24;
          const uint8_t *hb = p.high + row * p.high_row + g * 2;
          const _Float16 s = (_Float16)f16_to_f32(p.scale[row * p.groups + g]);
          const _Float16 zero = (_Float16)0.0f;
          // trits 30q..30q+29 from base bytes 6q..6q+5, then 120+2q, 121+2q
#pragma unroll
          for (int by = 0; by < 6; ++by) {
            uint32_t d[5];
            ptq1_digits(bb[6 * q + by], 5, d);
#pragma unroll
            for (int e = 0; e < 5; ++e)
              vals[5 * by + e] = d[e] == 0 ? -s : (d[e] == 1 ? zero : (d[e] == 2 ? s : (_Float16)(2.0f * (float)s)));
          }
          uint32_t dh[4];
          ptq1_digits(hb[q >> 1], 4, dh);
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const uint32_t dd = dh[2 * (q & 1) + e];
            vals[30 + e] = dd == 0 ? -s : (dd == 1 ? zero : s);
          }
        } else {
#pragma unroll
          for (int i = 0; i < 32; ++i) vals[i] = (_Float16)0.0f;
        }
        // natural k order inside the group: trits 30q.. and 120+2q..
        _Float16 *dst = &Bs[r * LDSROW];
#pragma unroll
        for (int e = 0; e < 30; ++e) dst[30 * q + e] = vals[e];
        dst[120 + 2 * q] = vals[30];
        dst[121 + 2 * q] = vals[31];
      }
    }
    __syncthreads();

    // ---- 8 k-steps of 16 on the matrix cores
#pragma unroll
    for (int ks = 0; ks < GK / 16; ++ks) {
      half8_t a[2], bfr[2];
      const int kb = ks * 16 + 8 * (lane >> 5);
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const half8_t *>(&As[(wm + 32 * i + (lane & 31)) * LDSROW + kb]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bfr[j] = *reinterpret_cast<const half8_t *>(&Bs[(wn + 32 * j + (lane & 31)) * LDSROW + kb]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }

  // ---- epilogue: D[i][j] of a 32x32 block sits in lane (j + 32*(i/4 % 2)),
  // value (i/8)*4 + i%4
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = n0 + wn + 32 * j + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = m0 + wm + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (row < M && col < p.n) {
          if constexpr (YD == DT_F32)
            static_cast<float *>(Y)[row * ldy + col] = acc[i][j][v];
          else
            static_cast<uint16_t *>(Y)[row * ldy + col] = f32_to_bf16(acc[i][j][v]);
        }
      }
    }
  }
}

template <int FMT, int XD>
static hipError_t gemm_go(const Planes &p, const uint16_t *x, int64_t m, int64_t ldx, void *y,
                          int yd, int64_t ldy, hipStream_t st) {
  const int tiles_n = (int)((p.n + GN - 1) / GN);
  const int tiles_m = (int)((m + GM - 1) / GM);
  dim3 grid((unsigned)(tiles_n * tiles_m)), block(256);
  if (yd == DT_F32)
    hipLaunchKernelGGL((gemm_kernel<FMT, XD, DT_F32>), grid, block, 0, st, p, x, m, ldx, y, ldy,
                       tiles_n, tiles_m);
  else
    hipLaunchKernelGGL((gemm_kernel<FMT, XD, DT_BF16>), grid, block, 0, st, p, x, m, ldx, y, ldy,
                       tiles_n, tiles_m);
  return hipGetLastError();
}

hipError_t launch_gemm(const Planes &p, const uint16_t *x, int xd, int64_t m, int64_t ldx, void *y,
                       int yd, int64_t ldy, hipStream_t st) {
  if (p.fmt == FMT_PQ2)
    return xd == DT_F16 ? gemm_go<FMT_PQ2, DT_F16>(p, x, m, ldx, y, yd, ldy, st)
                        : gemm_go<FMT_PQ2, DT_BF16>(p, x, m, ldx, y, yd, ldy, st);
  return xd == DT_F16 ? gemm_go<FMT_PTQ1, DT_F16>(p, x, m, ldx, y, yd, ldy, st)
                      : gemm_go<FMT_PTQ1, DT_BF16>(p, x, m, ldx, y, yd, ldy, st);
}

}  // namespace tq
