// The batch-1 decode GEMV with one wave per row (gfx950, wave64), shared by
// the row-split PQ2_0 planes and the expanded 2-bit G64 block stream: the two
// differ only in where a lane finds its codes and scales.
#pragma once

#include "tq_device.h"
#include "tq_launch.h"

#include <type_traits>

namespace tq {

__device__ __forceinline__ half2_t bits_h2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }

// The first products of the four accumulators, a[c] = t[c].lo*x[c].lo +
// t[c].hi*x[c].hi, each from a zero accumulator (three-operand form; the
// compiler only emits the two-operand form, whose accumulator is tied to the
// destination).  A dot product's result may be read by another vector
// instruction only three wait states later, which the compiler cannot see
// through the asm, so the block ends with those wait states itself.
__device__ __forceinline__ void dot2_first4(const uint32_t (&t)[8], const half2_t *x, float (&a)[4]) {
  asm("v_dot2_f32_f16 %0, %4, %8, 0\n\t"
      "v_dot2_f32_f16 %1, %5, %9, 0\n\t"
      "v_dot2_f32_f16 %2, %6, %10, 0\n\t"
      "v_dot2_f32_f16 %3, %7, %11, 0\n\t"
      "s_nop 2"
      : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3])
      : "v"(t[0]), "v"(t[1]), "v"(t[2]), "v"(t[3]),
        "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]));
}

// cache policy of a streaming (read-once) buffer load
constexpr int CPOL_NT = 2;

// Codes of one 16-weight dword as exact binary16 pairs.  Masked with
// 0x33333333, each nibble of the dword holds one code in its low two bits,
// which as an fp4 (E2M1) number is code/2; the converter with scale 2 turns
// byte B into the pair (code of nibble 2B, code of nibble 2B+1), i.e. the
// codes 0..3 as normal binary16 values.  The even codes (weights 4B, 4B+2)
// come from the dword itself, the odd ones (4B+1, 4B+3) from it shifted down
// two bits.  The codes stay normal numbers on purpose: the dot-product
// instruction keeps a product only down to a fixed absolute step of about
// 2^-38, so codes placed as binary16 subnormals (code * 2^-24) would lose
// the low bits of every product with a small activation.
template <int B>
__device__ __forceinline__ uint32_t codes_pair(uint32_t v) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, 2.0f, B));
}

// The eight code pairs of dword w, in the order the activation pairs are
// staged: pairs 0-3 = even weights (4B, 4B+2), pairs 4-7 = odd (4B+1, 4B+3).
__device__ __forceinline__ void dword_codes(uint32_t w, uint32_t (&t)[8]) {
  const uint32_t ev = w & 0x33333333u, od = (w >> 2) & 0x33333333u;
  t[0] = codes_pair<0>(ev); t[1] = codes_pair<1>(ev); t[2] = codes_pair<2>(ev); t[3] = codes_pair<3>(ev);
  t[4] = codes_pair<0>(od); t[5] = codes_pair<1>(od); t[6] = codes_pair<2>(od); t[7] = codes_pair<3>(od);
}

// Row layouts the kernel reads.
//  LAY_PLANES: PQ2_0_G128 row-split planes ([ninfer-skill] §3): a row's codes
//    are k/4 contiguous base bytes, its binary16 scales one per 128 weights
//    in the scale plane.
//  LAY_G64: the 2-bit G64 block stream ([tensorsharp] §4.1 expansion; block
//    rule of [gguf-explainer] §4.3): a row is k/64 blocks of 18 bytes, each
//    [binary16 d][16 code bytes] for 64 weights, with the same code order.
enum { LAY_PLANES = 0, LAY_G64 = 1 };

// What the kernel does around the product.
//  MODE_GEMV: x is the rotated activation row.
//  MODE_ROT:  x is unrotated; the kernel applies the signed transform.
//  MODE_HEAD: x is the last hidden row; the kernel applies RMSNorm with the
//             weight g and eps, then the signed transform, and reduces the
//             products (the logits) to the greedy token.
enum { MODE_GEMV = 0, MODE_ROT = 1, MODE_HEAD = 2 };

// Extra arguments of the fused modes.
//  MODE_HEAD: work[0] receives the running maximum of the (logit, index)
//    keys and the low word of work[1] counts finished workgroups; both are
//    zero before a launch and the last workgroup resets them after writing
//    the token.
//  MODE_ROT with tiles > 0: the transform input is x in the grouped head
//    order, element j taken from x[head_src(j)] (head_src below).
struct StepArgs {
  const uint16_t *g = nullptr;  // bf16 norm weight [k]
  float eps = 0.0f;
  unsigned long long *work = nullptr;
  int32_t *token = nullptr;
  int tiles = 0, groups = 0, head_dim = 0;
};

// Source position of transform-input element j in the grouped head order
// ([ninfer-skill] §5 perm_row, generalised): heads of head_dim elements, the
// target head h taken from source head (h % tiles) * groups + h / tiles.
// head_dim is a multiple of 16, so 16 consecutive elements from a multiple
// of 16 stay inside one head and move together.
__device__ __forceinline__ int head_src(int j, int tiles, int groups, int head_dim) {
  const int h = j / head_dim;
  return ((h % tiles) * groups + h / tiles) * head_dim + (j - h * head_dim);
}

// Order-preserving 64-bit key of (logit v, row i): the float's bits mapped
// so that unsigned order is numeric order (-0 is taken as +0), above the
// complement of the index, so that the maximum key is the largest logit
// with the lowest index.  A NaN logit is not ordered: its key is 0, the key
// of "no row", which every number (-inf included) beats, so a NaN is never
// the token and a head of NaN logits gives -1.
__device__ __forceinline__ unsigned long long greedy_key(float v, uint32_t i) {
  const uint32_t u = __float_as_uint(v + 0.0f);
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  const unsigned long long key = ((unsigned long long)o << 32) | (0xFFFFFFFFu - i);
  return v == v ? key : 0ull;
}

// The end of a head launch, on one thread per workgroup: the workgroup's
// largest key m goes into the launch's running maximum work[0], and the
// workgroup that finishes last (counted in the low word of work[1]) writes
// the token and zeroes both words.  The maximum is a returning atomic: its
// old value comes back only once the maximum has been performed where every
// workgroup's atomics meet, and the count is taken only after that value
// has arrived, so the last workgroup finds every other key in place.  No
// release or acquire ordering is needed for that; an agent-scope release
// would also write back this compute unit's dirty L2 lines (the logits) at
// every workgroup, which serialises the launch's end.
__device__ __forceinline__ void head_finish(unsigned long long m, unsigned long long *work, int32_t *token) {
  const unsigned long long old = __hip_atomic_fetch_max(&work[0], m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  asm volatile("" ::"v"(old) : "memory");  // the maximum has returned before the count
  uint32_t *done = reinterpret_cast<uint32_t *>(&work[1]);
  const uint32_t prev = __hip_atomic_fetch_add(done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (prev == gridDim.x - 1) {
    const unsigned long long k = __hip_atomic_load(&work[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    token[0] = (int32_t)(0xFFFFFFFFu - (uint32_t)k);
    __hip_atomic_store(&work[0], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ---------------------------------------------------------------------------
// Batch-1 GEMV, one wave per row.
//
// A row of k = 1024*m weights is cut into A = m/4 pieces of 4096 weights and
// BQ = m%4 pieces of 1024.  In a 4096-weight piece i lane l takes weights
// 4096i + 64l .. + 63 (planes: the 16 base bytes at 1024i + 16l, inside group
// 32i + l/2; G64: block 64i + l), in a 1024-weight piece j weights
// 4096A + 1024j + 16l .. + 15 (planes: the 4 bytes at 1024A + 256j + 4l,
// inside group 32A + 8j + l/8; G64: quarter l%4 of block 64A + 16j + l/4).
// Either way a lane's weights share one scale per piece.  Every load
// instruction of the wave covers one contiguous span, the wave's partial
// sums are reduced with lane swaps and DPP, and one lane writes each row:
// waves never synchronise, so each is an independent persistent stream over
// blocks of D consecutive rows (W = waves in the grid) with D rows in flight.
template <int LAY, int A, int BQ>
struct WRaw;

// planes: code dwords of the pieces, and their scale bits
template <int A, int BQ>
struct WRaw<LAY_PLANES, A, BQ> {
  uint32_t w[4 * A + BQ];
  uint32_t s[A + BQ];
};

// G64: five dwords per 4096-weight piece (the lane's block from a 4-byte
// boundary, scale included), two per 1024-weight piece and its scale bits
template <int A, int BQ>
struct WRaw<LAY_G64, A, BQ> {
  uint32_t w[5 * A + 2 * BQ];
  uint32_t s[BQ > 0 ? BQ : 1];
};

// Sums of up to 8 rows' per-lane partials v[0..D-1] over the 64 lanes of a
// wave, all at once: two swap stages halve the values per lane while pairing
// lane halves (32) and 16-lane rows, a rotate by 8 inside each 16-lane row
// merges the last two values, and three DPP row shifts finish each 8-lane
// group.  Lane 8g+7 then holds the total of row bitrev3(g); it is returned
// for that lane (other lanes return garbage) together with the row index.
template <int D>
__device__ __forceinline__ float rows8_sum(const float (&v)[D], int lane, int &row) {
  static_assert(D >= 1 && D <= 8, "at most 8 rows");
  auto bits = [](float f) { return __builtin_bit_cast(unsigned, f); };
  auto flt = [](unsigned u) { return __builtin_bit_cast(float, u); };
  float u[8];
#pragma unroll
  for (int d = 0; d < 8; ++d) u[d] = d < D ? v[d] : 0.0f;
  // lanes 0-31 | 32-63 of s1[i] carry rows 2i | 2i+1
  float s1[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const auto r = __builtin_amdgcn_permlane32_swap(bits(u[2 * i]), bits(u[2 * i + 1]), false, false);
    s1[i] = flt(r[0]) + flt(r[1]);
  }
  // 16-lane rows R0..R3 of s2[i] carry rows 4i + (0, 2, 1, 3)
  float s2[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const auto r = __builtin_amdgcn_permlane16_swap(bits(s1[2 * i]), bits(s1[2 * i + 1]), false, false);
    s2[i] = flt(r[0]) + flt(r[1]);
  }
  // lanes 0-7 of each 16-lane row keep s2[0], lanes 8-15 s2[1]; each adds
  // the matching value of the other half-row (row_ror:8)
  const bool hi = (lane & 8) != 0;
  const float keep = hi ? s2[1] : s2[0];
  const float give = hi ? s2[0] : s2[1];
  float x = keep + flt(__builtin_amdgcn_update_dpp(0u, bits(give), 0x128, 0xF, 0xF, false));
  x += flt(__builtin_amdgcn_update_dpp(0u, bits(x), 0x111, 0xF, 0xF, true));
  x += flt(__builtin_amdgcn_update_dpp(0u, bits(x), 0x112, 0xF, 0xF, true));
  x += flt(__builtin_amdgcn_update_dpp(0u, bits(x), 0x114, 0xF, 0xF, true));
  const int g = lane >> 3;
  row = ((g & 1) << 2) | (g & 2) | ((g >> 2) & 1);
  return x;
}

// Workgroups are fat (WPG waves, one workgroup per CU) because the
// activation row is read once per workgroup: every wave reading it on its own
// sends thousands of requests to the same few L2 lines.  The first NB waves
// ("staging" waves) stage it into LDS as binary16 pairs in the order the
// decoder consumes them, lane-major so that every lane later reads its own
// pairs with conflict-free 16-byte LDS reads.  The other waves request their first D weight rows as soon
// as the activations have arrived, so the weight stream runs while the
// staging waves work; the staging waves request theirs once the staging is
// done (a wave whose loads fill the compute unit's memory queue stalls at
// its next load until rows arrive, which would hold up the staging), unless
// every wave of the workgroup stages.
//
// MODE_ROT: the kernel also performs the signed transform of its input
// ([tensorsharp] §4.2: a projection input is rotated by H(D.x)/32 per
// 1024-element block): x is then the unrotated activation row, each staging
// wave transforms its 1024-element blocks in registers and rounds them to
// binary16 exactly as the standalone transform with binary16 output does,
// so one launch covers the whole step with the same result as two.
//
// MODE_HEAD: the output head of a decode step ([tensorsharp] §4.4: RMSNorm,
// signed transform, low-bit head, logits) with the greedy choice fused in
// (a GEMV that also finds the argmax, as [gguf-explainer] §4.5's drafter
// kernel does).  The transform is linear, so each staging wave transforms
// its blocks of x*g and the scalar 1/rms(x) is applied after it, once the
// staging waves have pooled their sums of squares (in a fixed order).  Each
// lane that holds a row's logit keeps the largest (logit, index) key, the
// workgroup takes the maximum over its waves, and one 64-bit atomic maximum
// per workgroup merges them; the last workgroup to finish writes the token.
// y (the logits) may be null.
template <int LAY, int A, int BQ, int D, int XD, int MODE, int WPG, int KS = 1>
__global__ __launch_bounds__(64 * WPG) void gemv_wave_kernel(Planes p, const void *__restrict__ x,
                                                             const uint16_t *__restrict__ signs,
                                                             float *__restrict__ y, StepArgs hd) {
  constexpr bool FUSED = MODE != MODE_GEMV;
  constexpr bool HEAD = MODE == MODE_HEAD;
  constexpr int NB = 4 * A + BQ;  // 1024-element blocks in a row = 16-weight dwords per lane
  constexpr int NP = A + BQ;      // pieces per lane
  // K split (KS = 2, long rows): the waves of a workgroup pair up, waves 2m
  // and 2m+1 sharing their rows.  Half 0 takes the first A/2 4096-weight
  // pieces of every row, half 1 the other A/2 and the 1024-weight pieces
  // (half 0 holds phantom copies of those: no bytes, zero activations).
  // Half 1 leaves its row sums in LDS; half 0 adds them to its own, in that
  // order, and writes the row.  Each wave then holds half the row's
  // activation pairs, so two waves fit a SIMD where one did.
  static_assert(KS == 1 || (KS == 2 && A % 2 == 0 && MODE != MODE_HEAD && WPG % 2 == 0),
                "the K split serves the GEMV (transform fused or not) with an even count of 4096-weight pieces");
  constexpr int AW = A / KS;        // 4096-weight pieces per wave
  constexpr int NBW = 4 * AW + BQ;  // code dwords (and activation dwords) per lane of a wave
  constexpr int NPW = AW + BQ;      // pieces per wave
  constexpr int KPASS = 8;          // passes per wave pair the row-sum slots hold (K split)
  __shared__ float kpart[KS == 2 ? WPG / 2 : 1][KS == 2 ? KPASS : 1][8];
  __shared__ uint32_t kready[KS == 2 ? WPG / 2 : 1];
  // Activation pairs: dword s of lane l (16 weights, pairs (4B, 4B+2) and
  // (4B+1, 4B+3) as dword_codes orders them) is held by quads (2s)*64 + l
  // (pairs 0-3) and (2s+1)*64 + l (pairs 4-7).  Dword s
  // of lane l is natural 16-element chunk 256i + 4l + d for s = 4i + d < 4A
  // (a kilobyte piece) and 256A + 64j + l for s = 4A + j (a 256-byte piece).
  __shared__ __attribute__((aligned(16))) u32x4 xq[NB * 128];
  __shared__ uint32_t staged;      // staging waves done
  __shared__ uint32_t sq_posted;   // HEAD: staging waves that posted their sum of squares
  __shared__ float sq_part[HEAD ? WPG : 1];
  __shared__ unsigned long long wbest[HEAD ? WPG : 1];
  // the transform's per-wave scratch (staging waves only)
  __shared__ __attribute__((aligned(16))) float wsc[FUSED ? (NB < WPG ? NB : WPG) : 1][WHT_SCRATCH];
  const int lane = threadIdx.x & 63;
  // the wave index is made explicitly uniform so that row offsets live in
  // scalar registers and every load is (scalar row base + lane offset)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kh = KS == 2 ? (wave & 1) : 0;  // the wave's half of every row
  const bool kmain = KS == 1 || kh == 1;    // the wave holds the 1024-weight pieces
  // row streams: one per wave, or one per wave pair
  const int64_t gw = KS == 2 ? (int64_t)blockIdx.x * (WPG / 2) + (wave >> 1) : (int64_t)blockIdx.x * WPG + wave;
  const int64_t W = (int64_t)gridDim.x * (WPG / KS);
  const bool stager = wave < NB;

  // ---- rows: in pass q wave gw takes the D consecutive rows (q*W + gw)*D
  // + d, so each wave streams one contiguous span of every plane; the launch
  // picks D so that every wave has the same share.  Slot loads are
  // unconditional: a branch around them would stop the compiler from
  // counting the loads still in flight, and it would then wait for all of
  // them at every row.  A slot whose next row lies past n re-reads the row
  // it already holds (fb), so such loads stay spread over the planes; the
  // last pass requests nothing (a wave cannot end before its loads return).
  // Row numbers are 32-bit (the launch guarantees n < 2^30): the scalar
  // unit has no 64-bit ordered compare, so 64-bit row tests would run on the
  // vector unit every row.
  const int n32 = (int)p.n;
  const int q0 = lane / 2, q1 = 32 * A + lane / 8;  // planes: scale entries
  // G64: a block is 18 bytes, so a 4096-weight piece is 1152 bytes and a
  // 1024-weight piece 288.  Lane l's block starts at 18l: 4-byte aligned for
  // even l (read 20 bytes from 18l: d, then the codes from byte 2) and 2 past
  // a boundary for odd l (read from 18l - 2: d in the high half of the first
  // dword, the codes dword aligned).  In a 1024-weight piece, quarter c of
  // block b holds its codes at 18b + 2 + 4c; 8 bytes read from 18b + 4c (b
  // even, codes at byte 2) or 18b + 4c - 2 (b odd, codes at byte 4) stay
  // inside the piece.  A byte permute with a per-lane selector then takes
  // each codes dword out of two neighbouring dwords.
  const int gb_off = 18 * lane - 2 * (lane & 1);
  const uint32_t gb_sel = (lane & 1) ? 0x07060504u : 0x05040302u;
  const int gb_sh = 16 * (lane & 1);
  const int gq_blk = lane >> 2;
  const int gq_off = 18 * gq_blk + 4 * (lane & 3) - 2 * (gq_blk & 1);
  const uint32_t gq_sel = (gq_blk & 1) ? 0x07060504u : 0x05040302u;
  auto load_row = [&](int row, int fb, WRaw<LAY, AW, BQ> &r) {
    const int rr = row < n32 ? row : fb;
    // the row's bytes as a buffer: the row address stays in scalar
    // registers and each load adds only the lane's offset (a streaming load
    // through a flat pointer would rebuild the 64-bit address every row)
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(p.base + (int64_t)rr * p.base_row), 0, (int)p.base_row, 0x00020000);
    if constexpr (LAY == LAY_PLANES) {
      const uint16_t *rs = p.scale + (int64_t)rr * p.groups;
#pragma unroll
      for (int i = 0; i < AW; ++i) {
        const int gi = i + AW * kh;  // the piece in the row
        const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(rb, 16 * lane + 1024 * gi, 0, CPOL_NT);
        r.w[4 * i] = t[0]; r.w[4 * i + 1] = t[1]; r.w[4 * i + 2] = t[2]; r.w[4 * i + 3] = t[3];
        r.s[i] = rs[q0 + 32 * gi];
      }
      // (phantoms read past the buffer's end: zero, and no bytes move)
#pragma unroll
      for (int j = 0; j < BQ; ++j) {
        r.w[4 * AW + j] = __builtin_amdgcn_raw_buffer_load_b32(
            rb, kmain ? 1024 * A + 4 * lane + 256 * j : 0x7FFFFFF0, 0, CPOL_NT);
        r.s[AW + j] = rs[q1 + 8 * j];
      }
    } else {
#pragma unroll
      for (int i = 0; i < AW; ++i) {
        const int gi = i + AW * kh;
        const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(rb, gb_off + 1152 * gi, 0, CPOL_NT);
        r.w[5 * i] = t[0]; r.w[5 * i + 1] = t[1]; r.w[5 * i + 2] = t[2]; r.w[5 * i + 3] = t[3];
        r.w[5 * i + 4] = __builtin_amdgcn_raw_buffer_load_b32(rb, gb_off + 1152 * gi + 16, 0, CPOL_NT);
      }
#pragma unroll
      for (int j = 0; j < BQ; ++j) {
        const int o = kmain ? 1152 * A + 288 * j : 0x7FFFF000;
        const u32x2 t = __builtin_amdgcn_raw_buffer_load_b64(rb, o + gq_off, 0, CPOL_NT);
        r.w[5 * AW + 2 * j] = t[0]; r.w[5 * AW + 2 * j + 1] = t[1];
        r.s[j] = __builtin_amdgcn_raw_buffer_load_b16(rb, o + 18 * gq_blk, 0, CPOL_NT);
      }
    }
  };
  // codes dword q of piece pc, and the piece's scale bits, of a loaded row
  auto codes_of = [&](const WRaw<LAY, AW, BQ> &r, int pc, int q) -> uint32_t {
    if constexpr (LAY == LAY_PLANES) {
      return r.w[pc < AW ? 4 * pc + q : 4 * AW + (pc - AW)];
    } else {
      if (pc < AW) return __builtin_amdgcn_perm(r.w[5 * pc + q + 1], r.w[5 * pc + q], gb_sel);
      return __builtin_amdgcn_perm(r.w[5 * AW + 2 * (pc - AW) + 1], r.w[5 * AW + 2 * (pc - AW)], gq_sel);
    }
  };
  // (a phantom piece's scale is zero)
  auto scale_of = [&](const WRaw<LAY, AW, BQ> &r, int pc) -> uint16_t {
    if constexpr (LAY == LAY_PLANES) return (KS == 1 || kmain || pc < AW) ? (uint16_t)r.s[pc] : (uint16_t)0;
    else return pc < AW ? (uint16_t)(r.w[5 * pc] >> gb_sh) : (uint16_t)r.s[pc - AW];
  };
  WRaw<LAY, AW, BQ> ring[D];
  const int gw32 = (int)gw, W32 = (int)W;
  const int first = gw32 * D < n32 ? gw32 * D : n32 - 1;
  auto load_first = [&]() {
#pragma unroll
    for (int d = 0; d < D; ++d) load_row(gw32 * D + d, first, ring[d]);
  };

  // ---- 1. the staging waves load the activations, and the workgroup
  // waits for them before any weight row is requested: requested alongside
  // the rows, they would queue behind the weight stream.  Fused: wave w
  // transforms blocks w, w + WPG, ... (chunks 64*block + lane); unfused:
  // thread t converts chunks t, t + 64*WPG, ...  Items past the end re-read
  // the last block or chunk, so the loads stay unconditional.
  constexpr int NI = FUSED ? (NB + WPG - 1) / WPG : (NB * 64 + 64 * WPG - 1) / (64 * WPG);
  Raw16<XD> xraw[NI];
  u32x4 sraw[FUSED ? NI : 1][2];
  u32x4 graw[HEAD ? NI : 1][2];
  auto item = [&](int i) -> int64_t {  // first element of item i of this thread
    if constexpr (FUSED) {
      const int blk = wave + WPG * i < NB ? wave + WPG * i : NB - 1;
      return (int64_t)blk * 1024 + 16 * lane;
    } else {
      const int c = (int)threadIdx.x + 64 * WPG * i;
      return 16 * (int64_t)(c < NB * 64 ? c : NB * 64 - 1);
    }
  };
  if (threadIdx.x == 0) {
    staged = 0;
    sq_posted = 0;
  }
  if (KS == 2 && threadIdx.x < WPG / 2) kready[threadIdx.x] = 0;
  if (stager) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if constexpr (MODE == MODE_ROT) {
        const int64_t e = item(i);
        load16_raw<XD>(x, hd.tiles ? (int64_t)head_src((int)e, hd.tiles, hd.groups, hd.head_dim) : e,
                       xraw[i]);
      } else {
        load16_raw<XD>(x, item(i), xraw[i]);
      }
      if constexpr (FUSED) {
        const u32x4 *sp = reinterpret_cast<const u32x4 *>(signs + item(i));
        sraw[i][0] = sp[0];
        sraw[i][1] = sp[1];
      }
      if constexpr (HEAD) {
        const u32x4 *gp = reinterpret_cast<const u32x4 *>(hd.g + item(i));
        graw[i][0] = gp[0];
        graw[i][1] = gp[1];
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  }
  __syncthreads();

  // ---- 2. the other waves request their first D rows now.  When every
  // wave stages (long rows, few waves), all of them do: the staging needs no
  // further global loads, so the rows stream in while it runs.
  constexpr bool ALL_STAGE = NB >= WPG;
  if (!stager || ALL_STAGE) load_first();
  __builtin_amdgcn_sched_barrier(0);

  // ---- 3. staging waves: activations -> binary16 pairs in LDS
  if (stager) {
    // HEAD: the scale of the norm, 1/sqrt(mean(x^2) + eps), folded with the
    // transform's 1/32; every staging wave posts the sum of squares of its
    // blocks, waits for the others and adds them in wave order
    float post = 0.03125f;
    if constexpr (HEAD) {
      constexpr uint32_t NSTG = NB < WPG ? NB : WPG;
      float sq = 0.0f;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        if (wave + WPG * i >= NB) continue;
        float v[16];
        convert16<XD>(xraw[i], v);
#pragma unroll
        for (int e = 0; e < 16; ++e) sq = __builtin_fmaf(v[e], v[e], sq);
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) sq += __shfl_xor(sq, o);
      if (lane == 0) sq_part[wave] = sq;
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      if (lane == 0) __hip_atomic_fetch_add(&sq_posted, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      for (int spin = 0; spin < (1 << 22); ++spin) {
        const uint32_t done = __builtin_amdgcn_readfirstlane(
            __hip_atomic_load(&sq_posted, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
        if (done >= NSTG) break;
        __builtin_amdgcn_s_sleep(1);
      }
      asm volatile("" ::: "memory");
      float tot = 0.0f;
#pragma unroll
      for (uint32_t w = 0; w < NSTG; ++w) tot += sq_part[w];
      post = 0.03125f / __builtin_sqrtf(tot / (float)(NB * 1024) + hd.eps);
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const bool mine = FUSED ? wave + WPG * i < NB : (int)threadIdx.x + 64 * WPG * i < NB * 64;
      if (!mine) continue;
      // h[m]: binary16 elements 2m, 2m+1 of this thread's 16-element chunk
      uint32_t h[8];
      if constexpr (FUSED) {
        float v[16];
        convert16<XD>(xraw[i], v);
        const uint32_t sw[8] = {sraw[i][0][0], sraw[i][0][1], sraw[i][0][2], sraw[i][0][3],
                                sraw[i][1][0], sraw[i][1][1], sraw[i][1][2], sraw[i][1][3]};
        if constexpr (HEAD) {
          const uint32_t gw[8] = {graw[i][0][0], graw[i][0][1], graw[i][0][2], graw[i][0][3],
                                  graw[i][1][0], graw[i][1][1], graw[i][1][2], graw[i][1][3]};
#pragma unroll
          for (int e = 0; e < 16; ++e) v[e] *= bf16_to_f32((uint16_t)(gw[e >> 1] >> (16 * (e & 1))));
        }
#pragma unroll
        for (int e = 0; e < 16; ++e)
          v[e] = apply_sign(v[e], (uint16_t)(sw[e >> 1] >> (16 * (e & 1))));
        // v[4g + j] leaves the transform holding element 256g + 4*lane + j
        // of the block; the block goes back through the wave's scratch in
        // natural order, and the lane takes chunk `lane` of it
        float *sc = wsc[wave];
        wht1024_wave(v, lane, sc);
        uint16_t *nat = reinterpret_cast<uint16_t *>(sc);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const uint32_t lo = (uint32_t)f32_to_f16(v[4 * g] * post) |
                              ((uint32_t)f32_to_f16(v[4 * g + 1] * post) << 16);
          const uint32_t hi = (uint32_t)f32_to_f16(v[4 * g + 2] * post) |
                              ((uint32_t)f32_to_f16(v[4 * g + 3] * post) << 16);
          *reinterpret_cast<u32x2 *>(nat + 256 * g + 4 * lane) = (u32x2){lo, hi};
        }
        const u32x4 *q = reinterpret_cast<const u32x4 *>(nat + 16 * lane);
        const u32x4 a0 = q[0], a1 = q[1];
        h[0] = a0[0]; h[1] = a0[1]; h[2] = a0[2]; h[3] = a0[3];
        h[4] = a1[0]; h[5] = a1[1]; h[6] = a1[2]; h[7] = a1[3];
      } else if constexpr (XD == DT_F16) {
#pragma unroll
        for (int m = 0; m < 4; ++m) { h[m] = xraw[i].q[0][m]; h[4 + m] = xraw[i].q[1][m]; }
      } else {
        float v[16];
        convert16<XD>(xraw[i], v);
#pragma unroll
        for (int m = 0; m < 8; ++m)
          h[m] = (uint32_t)f32_to_f16(v[2 * m]) | ((uint32_t)f32_to_f16(v[2 * m + 1]) << 16);
      }
      // pairs of the chunk in decode order: (4B, 4B+2) then (4B+1, 4B+3)
      uint32_t pr[8];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        pr[b] = __builtin_amdgcn_perm(h[2 * b + 1], h[2 * b], 0x05040100u);
        pr[4 + b] = __builtin_amdgcn_perm(h[2 * b + 1], h[2 * b], 0x07060302u);
      }
      const int c = FUSED ? (wave + WPG * i) * 64 + lane : (int)threadIdx.x + 64 * WPG * i;
      int s, l;
      if (c < 256 * A) {
        s = 4 * (c >> 8) + (c & 3);
        l = (c & 255) >> 2;
      } else {
        s = 4 * A + ((c - 256 * A) >> 6);
        l = (c - 256 * A) & 63;
      }
      xq[(2 * s) * 64 + l] = (u32x4){pr[0], pr[1], pr[2], pr[3]};
      xq[(2 * s + 1) * 64 + l] = (u32x4){pr[4], pr[5], pr[6], pr[7]};
    }
    // publish: the wave's LDS writes complete before the count (LDS
    // operations only: a release fence would also wait for the global loads)
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    if (lane == 0) __hip_atomic_fetch_add(&staged, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  // Every wave waits for all staging waves.  Not a workgroup barrier: the
  // other waves may still be stalled issuing their rows, and the staging
  // waves need not wait for that.  Each staging wave counts exactly once
  // on every path, so the wait ends; the bound only guards against a
  // defect turning into a hang.
  {
    constexpr uint32_t NSTG = NB < WPG ? NB : WPG;
    for (int spin = 0; spin < (1 << 22); ++spin) {
      const uint32_t done = __builtin_amdgcn_readfirstlane(
          __hip_atomic_load(&staged, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
      if (done >= NSTG) break;
      __builtin_amdgcn_s_sleep(1);
    }
    // the pair reads below are issued only after the count was seen, and
    // LDS executes them after the writes that preceded it
    asm volatile("" ::: "memory");
  }

  // ---- 4. the lane's activation pairs (read before the staging waves
  // request their rows, which may stall at issue)
  half2_t xp[NBW][8];
#pragma unroll
  for (int s = 0; s < NBW; ++s) {
    // the dword in the row's staging order, and whether it is a phantom
    const int sg = s < 4 * AW ? s + 4 * AW * kh : 4 * A + (s - 4 * AW);
    const bool ph = s >= 4 * AW && !kmain;
    const u32x4 a = xq[(2 * sg) * 64 + lane], b = xq[(2 * sg + 1) * 64 + lane];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      xp[s][k] = bits_h2(ph ? 0u : a[k]);
      xp[s][4 + k] = bits_h2(ph ? 0u : b[k]);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  if (stager && !ALL_STAGE) load_first();
  __builtin_amdgcn_sched_barrier(0);

  // sum over the lane's piece pc of code * x' for code words cw[0..nd-1],
  // in four accumulators (pair e feeds accumulator e % 4; the first product
  // of each starts from 0 instead of a zeroed register)
  auto piece_cx = [&](const uint32_t (&cw)[4], int pc) -> float {
    const int nd = pc < AW ? 4 : 1;
    const int d0 = pc < AW ? 4 * pc : 4 * AW + (pc - AW);
    float a[4];
#pragma unroll
    for (int q = 0; q < nd; ++q) {
      uint32_t t[8];
      dword_codes(cw[q], t);
      if (q == 0) dot2_first4(t, xp[d0], a);
#pragma unroll
      for (int e = q == 0 ? 4 : 0; e < 8; ++e)
        a[e & 3] = __builtin_amdgcn_fdot2(bits_h2(t[e]), xp[d0 + q][e], a[e & 3], false);
    }
    return (a[0] + a[1]) + (a[2] + a[3]);
  };
  // The offset of the code (trit = code - 1) is applied per piece as
  // s * (sum code*x' - xs).  xs is the same computation with every code 1,
  // the same instructions in the same order on the same activations, so a
  // piece whose weights are all zero gives cx == xs bit for bit and adds
  // exactly nothing: rounding error arises only in pieces that hold a
  // nonzero weight, and an all-zero row is exactly 0 at any scale.
  float xs[NPW];
  {
    const uint32_t ones[4] = {0x55555555u, 0x55555555u, 0x55555555u, 0x55555555u};
#pragma unroll
    for (int pc = 0; pc < NPW; ++pc) xs[pc] = piece_cx(ones, pc);
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- 5. passes of D rows
  unsigned long long best = 0;  // HEAD: the lane's largest key (0 is below every logit)
  int kpass = 0;                // K split: passes done
  auto do_pass = [&](int base, auto refill) {
    float part[D];
#pragma unroll
    for (int d = 0; d < D; ++d) {
      // sum over the lane's pieces of s * (sum code*x' - xs)
      float acc = 0.0f;
#pragma unroll
      for (int pc = 0; pc < NPW; ++pc) {
        const int nd = pc < AW ? 4 : 1;
        uint32_t cw[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int q = 0; q < nd; ++q) cw[q] = codes_of(ring[d], pc, q);
        acc += f16_to_f32(scale_of(ring[d], pc)) * (piece_cx(cw, pc) - xs[pc]);
      }
      part[d] = acc;
      // refill the slot with its row of the next pass
      if constexpr (decltype(refill)::value)
        load_row(base + d + D * W32, base + d < n32 ? base + d : n32 - 1, ring[d]);
      __builtin_amdgcn_sched_barrier(0);
    }
    int r;
    const float tot = rows8_sum<D>(part, lane, r);
    if constexpr (KS == 2) {
      // half 1 posts its row sums; half 0 waits for them (a bounded wait:
      // half 1 posts once per pass on every path) and writes the rows
      float(&slot)[8] = kpart[wave >> 1][kpass & (KPASS - 1)];
      if (kh == 1) {
        if ((lane & 7) == 7 && r < D) slot[r] = tot;
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        if (lane == 0)
          __hip_atomic_fetch_add(&kready[wave >> 1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      } else {
        for (int spin = 0; spin < (1 << 22); ++spin) {
          const uint32_t done = __builtin_amdgcn_readfirstlane(
              __hip_atomic_load(&kready[wave >> 1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
          if (done > (uint32_t)kpass) break;
          __builtin_amdgcn_s_sleep(1);
        }
        asm volatile("" ::: "memory");
        if ((lane & 7) == 7 && r < D && base + r < n32) y[base + r] = tot + slot[r];
      }
      ++kpass;
    } else if ((lane & 7) == 7 && r < D && base + r < n32) {
      if constexpr (HEAD) {
        if (y) y[base + r] = tot;
        const unsigned long long key = greedy_key(tot, (uint32_t)(base + r));
        best = key > best ? key : best;
      } else {
        y[base + r] = tot;
      }
    }
  };
  int base = gw32 * D;
  for (; base + D * W32 < n32; base += D * W32) do_pass(base, std::integral_constant<bool, true>{});
  if (base < n32) do_pass(base, std::integral_constant<bool, false>{});

  if constexpr (HEAD) {
    // the wave's maximum key, then the workgroup's, then one atomic maximum
    uint32_t hi = (uint32_t)(best >> 32), lo = (uint32_t)best;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const uint32_t ohi = (uint32_t)__shfl_xor((int)hi, o), olo = (uint32_t)__shfl_xor((int)lo, o);
      const bool take = ohi > hi || (ohi == hi && olo > lo);
      hi = take ? ohi : hi;
      lo = take ? olo : lo;
    }
    if (lane == 0) wbest[wave] = ((unsigned long long)hi << 32) | lo;
    __syncthreads();
    if (threadIdx.x == 0) {
      unsigned long long m = 0;
#pragma unroll
      for (int w = 0; w < WPG; ++w) m = wbest[w] > m ? wbest[w] : m;
      head_finish(m, hd.work, hd.token);
    }
  }
}

template <int LAY, int A, int BQ, int D, int XD, int MODE, int WPG>
static hipError_t gemv_wave_launch(const Planes &p, const void *x, const uint16_t *signs, float *y,
                                   const StepArgs &hd, int64_t waves, hipStream_t st) {
  const int64_t grid = (waves + WPG - 1) / WPG;
  hipLaunchKernelGGL((gemv_wave_kernel<LAY, A, BQ, D, XD, MODE, WPG>), dim3((unsigned)grid),
                     dim3(64 * WPG), 0, st, p, x, signs, y, hd);
  return hipGetLastError();
}

// Row split: for each ring depth D (D rows per wave and pass)
// take as many workgroups per CU as fit, the fewest passes that cover n, and
// then the fewest waves; keep the D whose busiest CU has the fewest rows
// (ties: the deeper ring).  Rows past n in a wave's last block re-read the
// row their slot already holds.  Workgroup size by register need: three
// waves per SIMD up to k = 5120 (WPG 12), two up to k = 7168 (WPG 8), one
// beyond (WPG 4).
template <int LAY, int A, int BQ, int D, int XD, int MODE, int WPG, int KS = 1>
static const void *gemv_wave_ptr() {
  return reinterpret_cast<const void *>(gemv_wave_kernel<LAY, A, BQ, D, XD, MODE, WPG, KS>);
}

// The K split for long rows (planes GEMV with four 4096-weight pieces, k =
// 16384 or 17408): eight waves, four pairs, per workgroup, so that two
// waves share a SIMD; the same row split as below over pairs, with at most
// eight passes a pair (the row-sum slots).  The fused transform needs k <=
// 11264, so the one-launch step never meets this form and keeps the
// two-launch result bit for bit.  done = false: no depth fits.
template <int LAY, int A, int BQ, int XD, int MODE>
static hipError_t gemv_wave_go_ks2(const Planes &p, const void *x, const uint16_t *signs, float *y,
                                   const StepArgs &hd, hipStream_t st, bool &done) {
  constexpr int WPG = 8, PAIRS = WPG / 2;
  const int depth[2] = {4, 5};
  const void *kerns[2] = {gemv_wave_ptr<LAY, A, BQ, 4, XD, MODE, WPG, 2>(),
                          gemv_wave_ptr<LAY, A, BQ, 5, XD, MODE, WPG, 2>()};
  const int cus = device_cus();
  int best = -1;
  int64_t best_rows = 0, best_wgs = 0;
  for (int i = 0; i < 2; ++i) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kerns[i], 64 * WPG, 0) != hipSuccess ||
        per_cu < 1)
      continue;
    const int64_t D = depth[i];
    const int64_t slots = (int64_t)PAIRS * cus * per_cu;
    const int64_t passes = (p.n + slots * D - 1) / (slots * D);
    if (passes > 8) continue;
    const int64_t pairs = (p.n + D * passes - 1) / (D * passes);
    const int64_t wgs = (pairs + PAIRS - 1) / PAIRS;
    const int64_t rows_cu = ((wgs + cus - 1) / cus) * PAIRS * D * passes;
    if (best < 0 || rows_cu <= best_rows) {
      best = i;
      best_rows = rows_cu;
      best_wgs = wgs;
    }
  }
  done = best >= 0;
  if (!done) return hipSuccess;
  if (depth[best] == 4)
    hipLaunchKernelGGL((gemv_wave_kernel<LAY, A, BQ, 4, XD, MODE, WPG, 2>), dim3((unsigned)best_wgs),
                       dim3(64 * WPG), 0, st, p, x, signs, y, hd);
  else
    hipLaunchKernelGGL((gemv_wave_kernel<LAY, A, BQ, 5, XD, MODE, WPG, 2>), dim3((unsigned)best_wgs),
                       dim3(64 * WPG), 0, st, p, x, signs, y, hd);
  return hipGetLastError();
}

template <int LAY, int A, int BQ, int XD, int MODE>
static hipError_t gemv_wave_go(const Planes &p, const void *x, const uint16_t *signs, float *y,
                               hipStream_t st, const StepArgs &hd = StepArgs{}) {
  constexpr int NBK = 4 * A + BQ;
  constexpr int WPG = NBK <= 5 ? 12 : NBK <= 7 ? 8 : 4;
  // (measured: 10.2 against 10.6 us at 5120 x 17408 and 9.1 against 9.6 at
  // 5120 x 16384; slower at k = 11264, where the halves hold 4096 and 7168
  // weights, and no faster on the G64 stream)
  if constexpr (LAY == LAY_PLANES && MODE == MODE_GEMV && A == 4) {
    bool done = false;
    const hipError_t e = gemv_wave_go_ks2<LAY, A, BQ, XD, MODE>(p, x, signs, y, hd, st, done);
    if (done) return e;
  }
  // ring depths tried: 4, 6, 8; the G64 stream also 5 (its long rows run
  // one wave per SIMD, where 5 rows per wave fill the chip at k = 17408)
  constexpr int ND = LAY == LAY_G64 ? 4 : 3;
  const int depth[4] = {4, 5, 6, 8};
  const void *kerns[4] = {gemv_wave_ptr<LAY, A, BQ, 4, XD, MODE, WPG>(), nullptr,
                          gemv_wave_ptr<LAY, A, BQ, 6, XD, MODE, WPG>(),
                          gemv_wave_ptr<LAY, A, BQ, 8, XD, MODE, WPG>()};
  if constexpr (LAY == LAY_G64) kerns[1] = gemv_wave_ptr<LAY, A, BQ, 5, XD, MODE, WPG>();
  const int cus = device_cus();
  int best = -1;
  int64_t best_rows = 0, best_waves = 0;
  for (int i = 0; i < 4; ++i) {
    if (!kerns[i] || (ND == 3 && depth[i] == 5)) continue;
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kerns[i], 64 * WPG, 0) != hipSuccess ||
        per_cu < 1)
      continue;  // this depth does not fit a workgroup on a CU
    const int64_t D = depth[i];
    const int64_t slots = (int64_t)WPG * cus * per_cu;
    const int64_t passes = (p.n + slots * D - 1) / (slots * D);
    const int64_t waves = (p.n + D * passes - 1) / (D * passes);
    const int64_t wgs = (waves + WPG - 1) / WPG;
    const int64_t rows_cu = ((wgs + cus - 1) / cus) * WPG * D * passes;
    if (best < 0 || rows_cu <= best_rows) {
      best = i;
      best_rows = rows_cu;
      best_waves = waves;
    }
  }
  if (best < 0) return hipErrorInvalidConfiguration;
  switch (depth[best]) {
    case 4: return gemv_wave_launch<LAY, A, BQ, 4, XD, MODE, WPG>(p, x, signs, y, hd, best_waves, st);
    case 6: return gemv_wave_launch<LAY, A, BQ, 6, XD, MODE, WPG>(p, x, signs, y, hd, best_waves, st);
    case 8: return gemv_wave_launch<LAY, A, BQ, 8, XD, MODE, WPG>(p, x, signs, y, hd, best_waves, st);
    default:
      if constexpr (LAY == LAY_G64)
        return gemv_wave_launch<LAY, A, BQ, 5, XD, MODE, WPG>(p, x, signs, y, hd, best_waves, st);
      return hipErrorInvalidConfiguration;
  }
}

}  // namespace tq
