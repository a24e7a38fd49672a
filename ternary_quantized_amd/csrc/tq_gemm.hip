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

// ---------------------------------------------------------------------------
// PQ2_0 prefill GEMM: 512-thread workgroups (8 waves), 64-deep K steps
// through two LDS stages, one barrier per step.
//
// Stage layout: X rows and decoded weight rows of [64 k + 8 pad] binary16.
// Inside every 16-wide k block both are stored in the k order
// (0,8,1,9,...,7,15): one dword of 16 codes decodes into the pairs (e, e+8),
// and X is permuted to match, so an MFMA k slot holds the same k in both
// operands.  Weights are decoded exactly with full-rate integer ops: the
// code ORed into the exponent field of 1024 gives 1024 + 4^e*code, one fma
// turns it into code - 1, and the product with the group scale is exactly 0
// or +-s.
//
// Register ring: while step s is multiplied, register set (s+1)&1 holds
// step s+1 (decoded and stored into the other stage between step s's MFMA
// slices) and set s&1 is refilled with step s+2, so each global load has a
// whole step to land.  The code loads are plain (cached) loads: one 128-byte
// line of a weight row serves 8 consecutive steps.
//
// Two tile shapes share the kernel: 256 x 256 tiles (waves 2 x 4 of 128 x
// 64) for the bulk, and 128 x 64 sub-tiles (waves 4 x 2 of 32 x 32) for the
// tiles of a last, partial round, which is split 8 ways so it fills the
// chip instead of a fraction of it.
constexpr int G2K = 64, G2ROW = G2K + 8;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t trit_pair_scaled(uint32_t t, float inv_m, float neg_c,
                                                     half2_t s2) {
  half2_t a = __builtin_bit_cast(half2_t, t), m, c;
  m.x = m.y = (_Float16)inv_m;
  c.x = c.y = (_Float16)neg_c;
  const half2_t trit = __builtin_elementwise_fma(a, m, c);  // exactly code - 1
  return __builtin_bit_cast(uint32_t, trit * s2);            // exactly 0 or +-s
}

// Half of a dword of 16 codes -> 4 binary16 pairs of t*s: part 0 gives the
// pairs (code e, code e+8) for e = 0..3, part 1 for e = 4..7.
template <int PART>
__device__ __forceinline__ void decode_pq2_ts4(uint32_t d, uint32_t magic, half2_t s2,
                                               uint32_t o[4]) {
  if constexpr (PART == 0) {
    o[0] = trit_pair_scaled((d & 0x00030003u) | magic, 1.0f, -1025.0f, s2);
    o[1] = trit_pair_scaled((d & 0x000C000Cu) | magic, 0.25f, -257.0f, s2);
    o[2] = trit_pair_scaled((d & 0x00300030u) | magic, 0.0625f, -65.0f, s2);
    o[3] = trit_pair_scaled((d & 0x00C000C0u) | magic, 0.015625f, -17.0f, s2);
  } else {
    const uint32_t d10 = d >> 10;
    o[0] = trit_pair_scaled((d & 0x03000300u) | magic, 0.00390625f, -5.0f, s2);
    o[1] = trit_pair_scaled((d10 & 0x00030003u) | magic, 1.0f, -1025.0f, s2);
    o[2] = trit_pair_scaled((d10 & 0x000C000Cu) | magic, 0.25f, -257.0f, s2);
    o[3] = trit_pair_scaled((d10 & 0x00300030u) | magic, 0.0625f, -65.0f, s2);
  }
}

template <int XD>
__device__ __forceinline__ uint32_t x_pair_f16(uint32_t v) {
  if constexpr (XD == DT_BF16) {
    const uint32_t lo = f32_to_f16(bf16_to_f32((uint16_t)(v & 0xFFFF)));
    const uint32_t hi = f32_to_f16(bf16_to_f32((uint16_t)(v >> 16)));
    return lo | (hi << 16);
  } else {
    return v;
  }
}

// One output tile of TM x TN at (m0, n0): waves WAVES_M x (8 / WAVES_M),
// each 32*FM x 32*FN.
template <int XD, int YD, int TM, int TN, int FM, int FN, int WAVES_M>
__device__ __forceinline__ void gemm_pq2_tile(const Planes &p, const uint16_t *__restrict__ X,
                                              int64_t M, int64_t ldx, void *__restrict__ Y,
                                              int64_t ldy, int64_t m0, int64_t n0,
                                              _Float16 *lds2) {
  constexpr int WAVES_N = 8 / WAVES_M;
  static_assert(WAVES_M * 32 * FM == TM && WAVES_N * 32 * FN == TN, "wave grid must cover the tile");
  constexpr int TPR = 512 / TM;       // threads per X row
  constexpr int HX = G2K / TPR;       // halves of X per thread and step
  constexpr int XQ = HX / 8;          // 16-byte X loads (and LDS writes) per thread and step
  static_assert(HX % 16 == 0 && XQ <= 4, "X share must be whole 16-wide k blocks");
  constexpr int STAGE = (TM + TN) * G2ROW;

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = (wave / WAVES_N) * 32 * FM, wn = (wave % WAVES_N) * 32 * FN;
  const int nsteps = (int)(p.k / G2K);  // even: k is a multiple of 128

  // X loads: row xr, halves [HX*xq, HX*xq + HX) of a step
  const int xr = t / TPR, xq = t % TPR;
  const bool xrow_ok = m0 + xr < M;
  const uint16_t *xsrc = X + (xrow_ok ? (m0 + xr) : 0) * ldx + HX * xq;
  // code loads (threads below 2*TN): row wr, codes [32*wh, 32*wh + 32) of a
  // step (8 bytes) and that row's group scale
  // (every thread loads codes when the tile is 256 wide: no branch, so the
  // compiler keeps counting the loads in flight instead of waiting for all
  // of them where a branch around a load would rejoin)
  const bool wthread = 2 * TN >= 512 || t < 2 * TN;
  const int wr = wthread ? t >> 1 : 0, wh = t & 1;
  const bool wrow_ok = wthread && n0 + wr < p.n;
  const int64_t wrow = wrow_ok ? n0 + wr : 0;
  const uint8_t *wsrc = p.base + wrow * p.base_row + 8 * wh;
  const uint16_t *ssrc = p.scale + wrow * p.groups;

  uint32_t xreg[2][HX / 2], wreg[4][2], sreg[4];
  auto clamp = [&](int st) { return st < nsteps ? st : nsteps - 1; };  // past the end: a harmless re-read
  auto load_x = [&](int set, int st) {
    const int64_t k0 = (int64_t)clamp(st) * G2K;
    const u32x4_t *q = reinterpret_cast<const u32x4_t *>(xsrc + k0);
#pragma unroll
    for (int i = 0; i < XQ; ++i) {
      const u32x4_t v = q[i];
#pragma unroll
      for (int c = 0; c < 4; ++c) xreg[set][4 * i + c] = v[c];
    }
  };
  auto load_w = [&](int set, int st) {
    if (wthread) {
      const int64_t k0 = (int64_t)clamp(st) * G2K;
      const u32x2_t w = *reinterpret_cast<const u32x2_t *>(wsrc + k0 / 4);
      wreg[set][0] = w[0];
      wreg[set][1] = w[1];
      sreg[set] = ssrc[k0 / 128];
    }
  };
  uint32_t magic = 0x64006400u;
  asm volatile("" : "+v"(magic));
  // quarter q of X set `set` and code set `wset` into an LDS stage: one
  // 16-byte write of permuted X (while q < XQ) and one of 8 decoded weights
  auto store_piece = [&](int set, int wset, int buf, int q) {
    _Float16 *As = lds2 + buf * STAGE;
    _Float16 *Bs = As + TM * G2ROW;
    if (q < XQ) {
      const uint32_t *xv = xreg[set] + 8 * (q >> 1) + 2 * (q & 1);
      uint32_t lo[2], hi[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        lo[c] = xrow_ok ? x_pair_f16<XD>(xv[c]) : 0u;
        hi[c] = xrow_ok ? x_pair_f16<XD>(xv[4 + c]) : 0u;
      }
      u32x4_t xo;
      xo[0] = __builtin_amdgcn_perm(hi[0], lo[0], 0x05040100u);
      xo[1] = __builtin_amdgcn_perm(hi[0], lo[0], 0x07060302u);
      xo[2] = __builtin_amdgcn_perm(hi[1], lo[1], 0x05040100u);
      xo[3] = __builtin_amdgcn_perm(hi[1], lo[1], 0x07060302u);
      *reinterpret_cast<u32x4_t *>(As + xr * G2ROW + HX * xq + 8 * q) = xo;
    }
    if (wthread) {
      const _Float16 sh = __builtin_bit_cast(_Float16, (uint16_t)sreg[wset]);
      half2_t s2;
      s2.x = s2.y = wrow_ok ? sh : (_Float16)0.0f;
      uint32_t o[4];
      if (q & 1)
        decode_pq2_ts4<1>(wreg[wset][q >> 1], magic, s2, o);
      else
        decode_pq2_ts4<0>(wreg[wset][q >> 1], magic, s2, o);
      *reinterpret_cast<u32x4_t *>(Bs + wr * G2ROW + 32 * wh + 8 * q) =
          (u32x4_t){o[0], o[1], o[2], o[3]};
    }
  };

  floatx16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // step s: X set s&1 is refilled with step s+2 and code set s&3 with step
  // s+4 (both already stored), stage s&1 is multiplied, and between its four
  // 16-deep k slices step s+1 (X set (s+1)&1, code set (s+1)&3) is stored
  // into the other stage.  Codes come from HBM, so they are fetched further
  // ahead; X mostly hits in L2.
  auto step = [&](int s, int ph) {  // ph = s & 3
    load_x(ph & 1, s + 2);
    load_w(ph, s + 4);
    const int buf = ph & 1;
    const _Float16 *As = lds2 + buf * STAGE;
    const _Float16 *Bs = As + TM * G2ROW;
    // operand fragments of slice ks+1 are read while slice ks is multiplied
    half8_t a[2][FM], bf[2][FN];
    auto frags = [&](int ks, int set) {
      const int kb = ks * 16 + 8 * (lane >> 5);
#pragma unroll
      for (int i = 0; i < FM; ++i)
        a[set][i] = *reinterpret_cast<const half8_t *>(As + (wm + 32 * i + (lane & 31)) * G2ROW + kb);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bf[set][j] = *reinterpret_cast<const half8_t *>(Bs + (wn + 32 * j + (lane & 31)) * G2ROW + kb);
    };
    frags(0, 0);
#pragma unroll
    for (int ks = 0; ks < G2K / 16; ++ks) {
      if (ks + 1 < G2K / 16) frags(ks + 1, (ks + 1) & 1);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[ks & 1][i], bf[ks & 1][j], acc[i][j],
                                                             0, 0, 0);
      store_piece((ph + 1) & 1, (ph + 1) & 3, buf ^ 1, ks);
    }
    __syncthreads();
  };

  load_x(0, 0);
  load_w(0, 0);
  load_x(1, 1);
#pragma unroll
  for (int i = 1; i < 4; ++i) load_w(i, i);
#pragma unroll
  for (int q = 0; q < 4; ++q) store_piece(0, 0, 0, q);
  __syncthreads();
  for (int s = 0; s < nsteps; s += 4) {  // nsteps is even
    step(s, 0);
    step(s + 1, 1);
    if (s + 2 < nsteps) {
      step(s + 2, 2);
      step(s + 3, 3);
    }
  }

  // epilogue: D[i][j] of a 32x32 block is in lane j + 32*((i/4) % 2),
  // element 4*(i/8) + i%4
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
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

// Work split of one launch over 256 x 256 tiles: workgroups [0, nbig) take
// whole tiles, the rest take 128 x 64 sub-tiles (8 per tile) of the tiles
// left over.  With `xcd` set, tiles are numbered band-major and XCD x (the
// workgroups b with b % 8 == x) owns the contiguous tiles [x*per,
// (x+1)*per), the first big_per of them whole; otherwise tiles go in plain
// order.
struct GemmSplit {
  int tiles_n;  // 256-wide tiles along N
  int per;      // tiles per XCD
  int big_per;  // whole tiles per XCD
  int nbig;     // workgroups on whole tiles
  int xcd;
};

template <int XD, int YD>
__global__ __launch_bounds__(512) void gemm_pq2_kernel(Planes p, const uint16_t *__restrict__ X,
                                                       int64_t M, int64_t ldx,
                                                       void *__restrict__ Y, int64_t ldy,
                                                       GemmSplit sp) {
  extern __shared__ __attribute__((aligned(16))) _Float16 lds2[];
  const int b = blockIdx.x;
  int tile, sub = -1;
  if (b < sp.nbig) {
    tile = sp.xcd ? (b % 8) * sp.per + b / 8 : b;
  } else {
    const int r = b - sp.nbig;
    if (sp.xcd) {
      const int s2 = r / 8;  // nbig is a multiple of 8, so r % 8 == b % 8
      tile = (r % 8) * sp.per + sp.big_per + s2 / 8;
      sub = s2 % 8;
    } else {
      tile = sp.nbig + r / 8;
      sub = r % 8;
    }
  }
  const int64_t m0 = (int64_t)(tile / sp.tiles_n) * 256, n0 = (int64_t)(tile % sp.tiles_n) * 256;
  if (sub < 0)
    gemm_pq2_tile<XD, YD, 256, 256, 4, 2, 2>(p, X, M, ldx, Y, ldy, m0, n0, lds2);
  else
    gemm_pq2_tile<XD, YD, 128, 64, 1, 1, 4>(p, X, M, ldx, Y, ldy, m0 + 128 * (sub >> 2),
                                            n0 + 64 * (sub & 3), lds2);
}

template <int XD, int YD>
static hipError_t gemm_pq2_go(const Planes &p, const uint16_t *x, int64_t m, int64_t ldx, void *y,
                              int64_t ldy, hipStream_t st) {
  GemmSplit sp;
  sp.tiles_n = (int)((p.n + 255) / 256);
  const int total = sp.tiles_n * (int)((m + 255) / 256);
  const int cus = device_cus();
  // a last round that would occupy at most 1/8 of the CUs is split 8 ways
  const int left = total % cus;
  const bool split = total > cus && left > 0 && 8 * left <= cus;
  sp.xcd = total % 8 == 0 && (!split || left % 8 == 0);
  if (sp.xcd) {
    sp.per = total / 8;
    sp.big_per = split ? sp.per - left / 8 : sp.per;
    sp.nbig = 8 * sp.big_per;
  } else {
    sp.per = sp.big_per = 0;
    sp.nbig = split ? total - left : total;
  }
  const int grid = sp.nbig + 8 * (total - sp.nbig);
  const size_t lds = (size_t)2 * (256 + 256) * G2ROW * sizeof(_Float16);
  auto kern = gemm_pq2_kernel<XD, YD>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(512), lds, st, p, x, m, ldx, y, ldy, sp);
  return hipGetLastError();
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
  // PQ2_0 with k a multiple of the 64-deep step: the pipelined 256x256 kernel
  if (p.fmt == FMT_PQ2 && p.k % G2K == 0) {
    if (xd == DT_F16)
      return yd == DT_F32 ? gemm_pq2_go<DT_F16, DT_F32>(p, x, m, ldx, y, ldy, st)
                          : gemm_pq2_go<DT_F16, DT_BF16>(p, x, m, ldx, y, ldy, st);
    return yd == DT_F32 ? gemm_pq2_go<DT_BF16, DT_F32>(p, x, m, ldx, y, ldy, st)
                        : gemm_pq2_go<DT_BF16, DT_BF16>(p, x, m, ldx, y, ldy, st);
  }
  if (p.fmt == FMT_PQ2)
    return xd == DT_F16 ? gemm_go<FMT_PQ2, DT_F16>(p, x, m, ldx, y, yd, ldy, st)
                        : gemm_go<FMT_PQ2, DT_BF16>(p, x, m, ldx, y, yd, ldy, st);
  return xd == DT_F16 ? gemm_go<FMT_PTQ1, DT_F16>(p, x, m, ldx, y, yd, ldy, st)
                      : gemm_go<FMT_PTQ1, DT_BF16>(p, x, m, ldx, y, yd, ldy, st);
}

}  // namespace tq
