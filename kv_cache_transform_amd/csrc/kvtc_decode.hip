// HIP kernels of the decompression side of KV-cache transform coding for
// gfx950 (MI355X): the two-stage decode and the kvtc_unpack test hook.
//
// Method: "KV Cache Transform Coding for Compact Storage in LLM Inference"
// (gist.science, 2511.01815), section 2C: dequantize, multiply by V^T, add
// the mean, layer by layer.
//
// Stage 1 (256 threads): one wave per block of 32 compressed tokens loads
// the block's records, stages them in LDS and builds each token's dequantized
// coefficients c_hat = shift + q * fp32(scale / k) for the 8 components per K
// step it feeds to the MFMA, divided by a per-token power of two into fp16
// (the fp16 operand keeps 11 significant bits; the scale makes the range
// irrelevant), into a staging buffer. Stage 2 (512 threads, persistent):
// D[feature][token] = sum_j V'[feature][j] * c_hat[token][j] on
// v_mfma_f32_32x32x16_f16 per 128-feature slab (V' in LDS), written as
// S_t * D + mu through LDS rows in coalesced row-piece stores.
#include <mutex>

#include "kvtc_device.h"

namespace kvtc {

// --------------------------------------------------------------- decode ---
//
// Decode runs in two kernels. Stage 1 (prep) turns each token's record into
// the MFMA B operands of the reconstruction: the dequantized coefficients
// c_hat / S_t as fp16, in MFMA lane order, with S_t a per-token power of two,
// written to a staging buffer. Stage 2 (gemm) computes x_hat = S_t * (V' B) +
// mu for every compressed row, a tall-skinny product whose cost is writing
// the output. Dequantizing once per token in stage 1 keeps that work out of
// stage 2, whose tiles each cover a slab of features.

// Per-token power-of-two scale: S = 2^(e - 14) where 2^e <= max |c_hat| over
// the token's groups < 2^(e+1), so the fp16 operand peaks in [2^14, 2^15).
__device__ __forceinline__ void token_scale(float m, float& S, float& Sinv) {
  int e = (int)((__float_as_uint(m) >> 23) & 0xFF) - 127;
  if (m == 0.f) e = 14;
  e = max(min(e, 100), -100);
  S = __uint_as_float((uint32_t)(127 + e - 14) << 23);
  Sinv = __uint_as_float((uint32_t)(127 + 14 - e) << 23);
}

// fp32(scale / k) for k = 2^w - 1 from rk = fp32(1 / k): the product and one
// fma correction (the residual scale - q k is exact in an fma), which gives
// the correctly rounded quotient except in rare double-rounding cases, and
// exactly whenever the quotient is representable (the decode tolerance does
// not depend on the last bit; both decode routes share this function).
__device__ __forceinline__ float div_by_levels(float scale, float kf, float rk) {
  const float q = scale * rk;
  return __builtin_fmaf(__builtin_fmaf(-q, kf, scale), rk, q);
}

// B fragment of 8 components of a group of width W from packed record bits
// (code j at bits [j W, j W + W), LSB first): c_hat = shift + q * step,
// step = fp32(scale / k), times the power of two Sinv, as packed fp16.
// Sinv is folded into the fma operands; scaling by a power of two is exact,
// so the rounded results are those of the unscaled fma times Sinv. The bit
// offsets are constants, so each code is one field extract (two where it
// straddles the 32-bit halves).
template <int W>
__device__ __forceinline__ uint4 frag_w(uint64_t bits, float step, float sh) {
  uint32_t v[8];
  codes8_w<W>(bits, v);
  uint32_t pk[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    pk[j] = pack_f16x2(__builtin_fmaf((float)v[2 * j], step, sh), __builtin_fmaf((float)v[2 * j + 1], step, sh));
  return make_uint4(pk[0], pk[1], pk[2], pk[3]);
}

// codes8_w for a width w in 1..8 known only at run time (uniform).
__device__ __forceinline__ void codes8(uint64_t bits, int w, uint32_t (&v)[8]) {
  switch (w) {
    case 1: codes8_w<1>(bits, v); break;
    case 2: codes8_w<2>(bits, v); break;
    case 3: codes8_w<3>(bits, v); break;
    case 4: codes8_w<4>(bits, v); break;
    case 5: codes8_w<5>(bits, v); break;
    case 6: codes8_w<6>(bits, v); break;
    case 7: codes8_w<7>(bits, v); break;
    default: codes8_w<8>(bits, v); break;
  }
}

// The same for a width w in 1..8 known only at run time (uniform across the
// wave: one branch per fragment); kf = 2^w - 1 and rk = fp32(1 / kf).
__device__ __forceinline__ uint4 frag_from_bits(uint64_t bits, float shift, float scale, int w,
                                                float kf, float rk, float Sinv) {
  const float step = div_by_levels(scale, kf, rk) * Sinv;
  const float sh = shift * Sinv;
  switch (w) {
    case 1: return frag_w<1>(bits, step, sh);
    case 2: return frag_w<2>(bits, step, sh);
    case 3: return frag_w<3>(bits, step, sh);
    case 4: return frag_w<4>(bits, step, sh);
    case 5: return frag_w<5>(bits, step, sh);
    case 6: return frag_w<6>(bits, step, sh);
    case 7: return frag_w<7>(bits, step, sh);
    default: return frag_w<8>(bits, step, sh);
  }
}

// B fragment of 8 components with a width each (a width per component):
// entry = (bit position in the record << 8) | width; c_hat = shift + q *
// fp32(scale / k) times the power of two Sinv as in frag_from_bits, and 0
// for a zero width. A code spans at most two bytes of the record row.
__device__ __forceinline__ uint4 frag_pc(const uint8_t* rec, const uint32_t* ent, float shift, float scale,
                                         float Sinv) {
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t e = ent[i], pos = e >> 8;
    const int w = (int)(e & 0xFFu);
    x[i] = 0.f;
    if (w) {
      const uint32_t b2 = (uint32_t)rec[pos >> 3] | ((uint32_t)rec[(pos >> 3) + 1] << 8);
      const uint32_t q = (b2 >> (pos & 7u)) & ((1u << w) - 1u);
      const float kf = (float)((1 << w) - 1);
      x[i] = __builtin_fmaf((float)q, div_by_levels(scale, kf, 1.0f / kf) * Sinv, shift * Sinv);
    }
  }
  return make_uint4(pack_f16x2(x[0], x[1]), pack_f16x2(x[2], x[3]), pack_f16x2(x[4], x[5]),
                    pack_f16x2(x[6], x[7]));
}

// Stage 1, one launch over a batch of jobs. First the header and
// passthrough units (kPrepPassRows rows each; job j owns max(1, units) of
// them from cblk_begin, and its first one records the header check in the
// job's status word), split evenly over the workgroups so they add little to
// any one; then one wave per block of kDecTok compressed tokens (block
// tile_begin + c of job j is the c-th block of its records): the wave loads
// the block's records with coalesced 16-byte loads (all in flight at once),
// stores them into its LDS rows (stride rb + 16 if rb % 16 == 0, which keeps
// a vector inside one row and spreads the rows over the banks; contiguous
// otherwise), and builds the B operands and token scales of its 32 tokens,
// stg_block_bytes(KS) bytes of staging per block. No workgroup barrier
// follows the passthrough units: the waves run on their own.
// PC: every job of the launch has a width per component (frag_pc).
template <int KS, bool PC>
__global__ __launch_bounds__(kThreads) void prep_kernel(const LaunchArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ int flag;
  constexpr int KA = KS > 0 ? KS : 1;
  // 16-byte record vectors per lane for a block of the widest record this
  // K-step count allows (every active group of width <= 8 adds at most
  // 8 + G bytes per G / 16 K steps: rb <= 24 KS).
  constexpr int NV = (kDecTok * 24 * KA / 16 + 63) / 64;
  const uint32_t g = logical_tile(), ng = gridDim.x;
  {
    const uint32_t P = a.total_cblks;
    const uint32_t p_end = (uint32_t)((uint64_t)P * (g + 1) / ng);
    for (uint32_t p = (uint32_t)((uint64_t)P * g / ng); p < p_end; ++p) {
      const JobDesc& jd = a.jobs[job_at<&JobDesc::cblk_begin>(a, p)];
      CSlot& sl = slot_of(a, jd.slot);
      const uint32_t lp = p - jd.cblk_begin;
      const int st = check_header(a, jd, sl);   // uniform
      if (lp == 0 && threadIdx.x == 0) set_status(a, jd.status_idx, st);
      if (st != KVTC_OK) continue;
      if (threadIdx.x == 0) flag = 0;
      __syncthreads();
      bool ok = true;
      if (lp * kPrepPassRows < jd.s1 + jd.w1)
        ok = decode_passthrough<kThreads, kPrepPassRows>(a, jd, lp, (long*)smem);
      if (!ok) atomicExch(&flag, 1);
      __syncthreads();
      if (threadIdx.x == 0 && flag) set_status(a, jd.status_idx, KVTC_E_INVALID);
      __syncthreads();   // row list and flag are free for the next unit
    }
  }
  const int lane = threadIdx.x & 63, t = lane & 31, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const uint32_t b = g * kWaves + wave;
  if (b >= a.total_tiles || KS == 0) return;
  const int j = find_job(a, b);
  const JobDesc& jd = a.jobs[j];
  CSlot& sl = slot_of(a, jd.slot);
  if (check_header(a, jd, sl) != KVTC_OK) return;   // reported by the job's first unit
  const uint32_t c = b - jd.tile_begin;
  const uint32_t nrec = min((uint32_t)kDecTok, jd.tc - c * kDecTok);
  const int rb = sl.record_bytes, rbp = dec_rec_stride(rb);
  // row of record byte q: (q * mrb) >> 24 = q / rb exactly for q < 2^24 / rb
  const uint32_t mrb = (0xFFFFFFu + (uint32_t)rb) / (uint32_t)rb;
  const uint32_t nbytes = nrec * (uint32_t)rb, nvv = nbytes / 16u;
  const uint8_t* rec = (const uint8_t*)jd.src + record_base(jd, a.F, a.dtype == KVTC_F32 ? 4 : 2) +
                       (size_t)c * kDecTok * rb;
  uint8_t* rows = smem + kPrepRowsOff + (size_t)wave * a.wave_lds;
  u32x4 x[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i)
    if ((uint32_t)(64 * i) < nvv)   // uniform
      x[i] = *(const u32x4*)(rec + (size_t)min((uint32_t)(lane + 64 * i), nvv - 1u) * 16);
  // Byte q of the block's records goes to LDS byte q + (q / rb) * (rbp - rb).
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const uint32_t q = (uint32_t)(lane + 64 * i) * 16u;
    if ((uint32_t)(64 * i) < nvv && q < nbytes - 15u)
      *(u32x4*)(rows + q + ((q * mrb) >> 24) * (uint32_t)(rbp - rb)) = x[i];
  }
  for (uint32_t q = nvv * 16u + lane; q < nbytes; q += 64) rows[q] = rec[q];   // ragged end (rbp == rb)
  wave_lds_sync();
  // K step s: components 16 s + 8 h .. + 8 of active group ag = 16 s / G
  // (both halves lie in one group since G >= 16, so the group, its width and
  // the reciprocal of its level count are uniform); their w-bit codes start at
  // byte off of the record, the group's (shift, scale) at byte 8 ag.
  const bool tok_ok = (uint32_t)t < nrec;
  const uint8_t* r = rows + (tok_ok ? t : 0) * rbp;
  const int G = sl.G;
  float2 ps[KA];
  float m = 0.f;
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    ps[s] = get_scales(r, 16 * s / G);   // rows are 2-byte aligned
    // every active group has a component among the K steps, so both lanes
    // of a token see the same maximum
    m = fmaxf(m, fmaxf(fabsf(ps[s].x), fabsf(ps[s].x + ps[s].y)));
  }
  float S, Sinv;
  token_scale(m, S, Sinv);
  uint8_t* blk = (uint8_t*)jd.staging + (size_t)c * stg_block_bytes(KS);
  const uint32_t* pcw = PC ? (const uint32_t*)(a.state + sl.pcw_off) : nullptr;
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const int ag = 16 * s / G;
    uint4 f = make_uint4(0u, 0u, 0u, 0u);
    if (PC) {
      if (tok_ok) f = frag_pc(r, pcw + 16 * s + 8 * h, ps[s].x, ps[s].y, Sinv);
    } else {
      const int w = slot_width(sl, ag);
      const float kf = (float)((1 << w) - 1);
      if (tok_ok)
        f = frag_from_bits(code_bits8(r, sl, ag, 16 * s + 8 * h - ag * G, w), ps[s].x, ps[s].y, w, kf,
                           1.0f / kf, Sinv);
    }
    *(uint4*)(blk + s * 1024 + lane * 16) = f;
  }
  if (h == 0) *(float*)(blk + KS * 1024 + t * 4) = tok_ok ? S : 1.f;
}

// ------------------------------------------------------- restore kernel ---
//
// Restore: x_hat = S_t * (V' B) + mu for every compressed row, where B holds
// the token's dequantized coefficients c_hat / S_t as fp16 MFMA operands.
// It is decode stage 2 (B from the staging stage 1 wrote) and, FUSED, the
// whole decode (headers, passthrough rows, and B built here from the
// records, with the arithmetic of stage 1).
//
// 512 threads (8 waves), one workgroup per CU, persistent over an equal
// contiguous range of units; a unit is one block of kDecTok compressed tokens
// of one slab of rest_slab(NFB) features of one job, units ordered (job,
// slab, block). Wave w owns features [f0 + 32 NFB w, + 32 NFB) of the slab
// and holds their V' fragments (NFB x KS of them, fp16) in registers while
// its units share (job, slab), so a workgroup writes whole output rows (at
// F = 1024 and NFB = 4, 2 KB per row, 64 KB per block) and each token is
// dequantized once.
//
// Per unit u the workgroup runs one barrier-separated step of a pipeline
// over LDS buffers (three fragment buffers in rotation, two record buffers
// by unit parity):
//   FUSED: the records of unit u + 2 are loaded into registers (16-byte
//     loads); unit u - 1, whose product is still in the accumulators, is
//     staged and stored while unit u's MFMAs run between its stores, and
//     waves 0 .. KS - 1 build the B fragments and token scales of unit u + 1
//     (one K step each) from its records between the stores too; the loaded
//     records then go to the record buffer unit u + 1 does not use;
//   not FUSED: the staging block of unit u + 1 is loaded into the next
//     fragment buffer, with the same stores and MFMAs.
// Deferring each unit's stores to the next step keeps every wave issuing
// stores from the start of a step, with this step's other work between them,
// instead of computing first and storing last.
// Compute: B fragments from LDS, NFB x KS MFMAs D[feature][token]
// (v_mfma_f32_32x32x16_f16, K-step-outer so consecutive MFMAs go to
// different accumulators), S_t * D + mu through the wave's LDS staging rows,
// then coalesced 16-byte stores of 256-byte row pieces. Every wave
// issues the same loads and stores for every unit (addresses are clamped to
// valid ones, rows without a destination go to the workspace sink), so the
// wait for the next unit's loads, issued before these stores, never covers
// them.

struct RUnit {
  int j;              // job, -1 past the workgroup's range
  uint32_t slab, c;   // feature slab, block of the job's compressed rows
  uint32_t nrec;      // compressed tokens in the block
  uint32_t n_ch;      // blocks of the job
  uint32_t left;      // units of the range from this one on (0: past it)
};

// Unit u of the launch (a search over the jobs and a division: once per
// workgroup); rest_next steps to the following unit without either.
__device__ __forceinline__ RUnit rest_unit_at(const LaunchArgs& a, uint32_t u, uint32_t u_hi) {
  RUnit r;
  r.left = u < u_hi ? u_hi - u : 0u;
  if (!r.left) {
    r.j = -1;
    r.slab = r.c = r.nrec = r.n_ch = 0;
    return r;
  }
  const int j = job_at<&JobDesc::tile_begin>(a, u);
  const JobDesc& jd = a.jobs[j];
  r.j = j;
  r.n_ch = (jd.tc + kDecTok - 1) / kDecTok;
  const uint32_t lu = u - jd.tile_begin;
  r.slab = lu / r.n_ch;
  r.c = lu - r.slab * r.n_ch;
  r.nrec = min((uint32_t)kDecTok, jd.tc - r.c * kDecTok);
  return r;
}
__device__ __forceinline__ RUnit rest_next(const LaunchArgs& a, RUnit r, uint32_t n_slabs) {
  if (r.left <= 1) {
    r.left = 0;
    r.j = -1;
    return r;
  }
  --r.left;
  if (++r.c == r.n_ch) {
    r.c = 0;
    if (++r.slab == n_slabs) {
      r.slab = 0;
      do {   // the range still has units, so a job with rows follows
        ++r.j;
      } while (a.jobs[r.j].n_ctiles == 0);
      r.n_ch = (a.jobs[r.j].tc + kDecTok - 1) / kDecTok;
    }
  }
  r.nrec = min((uint32_t)kDecTok, a.jobs[r.j].tc - r.c * kDecTok);
  return r;
}

// Output row of the block's token i (lanes < 32), for the unit's job: >= 0
// a row of dst, -1 past the job's compressed rows, -2 a bad block table
// entry. The block table is read for every thread (index 0 where there is no
// token), so all threads issue the same load.
__device__ __forceinline__ int rest_row_entry(const JobDesc& jd, uint32_t c, int i, int& ent) {
  const uint32_t tok = c * kDecTok + (uint32_t)i;
  const bool in = i < kDecTok && tok < jd.tc;
  const uint32_t tt = jd.s1 + tok;
  const uint32_t bi = in ? (jd.bs_shift >= 0 ? tt >> jd.bs_shift : tt / (uint32_t)jd.block_size) : 0u;
  ent = jd.block_table[bi];
  return in ? 1 : 0;
}
__device__ __forceinline__ int rest_row(const JobDesc& jd, uint32_t c, int i, int in, int ent) {
  if (!in) return -1;
  if (ent < 0 || ent >= jd.n_blocks) return -2;
  const uint32_t tt = jd.s1 + c * kDecTok + (uint32_t)i;
  const uint32_t in_blk = jd.bs_shift >= 0 ? tt & ((1u << jd.bs_shift) - 1u) : tt % (uint32_t)jd.block_size;
  return ent * jd.block_size + (int)in_blk;
}

// Rows of dst a store may address: n_blocks * block_size (the host checks
// them against dst_capacity), or T for a contiguous job (one block of 2^30
// rows through a zero entry).
__device__ __forceinline__ uint32_t rest_row_limit(const JobDesc& jd) {
  return jd.n_blocks == 1 && jd.block_size == (1 << 30) ? jd.T : (uint32_t)jd.n_blocks * (uint32_t)jd.block_size;
}

// Epilogue staging of one round of FBR feature blocks (32 features each,
// starting at block fb0): S_t * D + mu into the wave's staging rows, RB =
// FBR * 32 * OSZ bytes per row, as 16-byte chunks: logical chunk q of row t
// at chunk q ^ (t & 7). Every lane writes whole chunks (ds_write_b128), and
// the swizzle sends the 8 lanes an LDS cycle serves (8 rows, one logical
// chunk) to 8 different bank groups; the stores read each row's chunks back
// in 16-lane groups, which the swizzle only permutes.
// MFMA D[feature][token] leaves lane (t, h) with features 8 qd + 4 h + 0..3
// of token t per qd. For f32 output that is one chunk. For bf16 the lane
// halves trade packed values (v_permlane32_swap) so that lane (t, 0) holds
// features 16 p + 0..7 and lane (t, 1) features 16 p + 8..15 of qd pair p.
template <int OSZ, int FBR, int NFB>
__device__ __forceinline__ void rest_stage(const f32x16 (&acc)[NFB], int fb0, float S, const float* mu_w,
                                           uint8_t* stg) {
  constexpr int RB = FBR * 32 * OSZ;
  const int lane = threadIdx.x & 63, t = lane & 31, h = lane >> 5;
  uint8_t* row = stg + t * RB;
  const int sw = t & 7;
#pragma unroll
  for (int f = 0; f < FBR; ++f) {
    const f32x16& a = acc[fb0 + f];
    const float* mu_f = mu_w + 32 * (fb0 + f);
    if (OSZ == 4) {
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const float4 m4 = *(const float4*)(mu_f + 8 * qd + 4 * h);
        const float4 o = make_float4(__builtin_fmaf(a[4 * qd + 0], S, m4.x), __builtin_fmaf(a[4 * qd + 1], S, m4.y),
                                     __builtin_fmaf(a[4 * qd + 2], S, m4.z), __builtin_fmaf(a[4 * qd + 3], S, m4.w));
        const int q = 8 * f + 2 * qd + h;
        *(float4*)(row + (q ^ sw) * 16) = o;
      }
    } else {
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        // qd 2p in acc[8p .. 8p+3], qd 2p+1 in acc[8p+4 .. 8p+7]
        const float4 ma = *(const float4*)(mu_f + 16 * p + 4 * h);
        const float4 mb = *(const float4*)(mu_f + 16 * p + 8 + 4 * h);
        const uint32_t p0 = pack_bf16x2(__builtin_fmaf(a[8 * p + 0], S, ma.x), __builtin_fmaf(a[8 * p + 1], S, ma.y));
        const uint32_t p1 = pack_bf16x2(__builtin_fmaf(a[8 * p + 2], S, ma.z), __builtin_fmaf(a[8 * p + 3], S, ma.w));
        const uint32_t q0 = pack_bf16x2(__builtin_fmaf(a[8 * p + 4], S, mb.x), __builtin_fmaf(a[8 * p + 5], S, mb.y));
        const uint32_t q1 = pack_bf16x2(__builtin_fmaf(a[8 * p + 6], S, mb.z), __builtin_fmaf(a[8 * p + 7], S, mb.w));
        // lanes 0-31 keep p* and take the upper lanes' p*; lanes 32-63
        // take the lower lanes' q* and keep q*
        const auto x = __builtin_amdgcn_permlane32_swap(p0, q0, false, false);
        const auto y = __builtin_amdgcn_permlane32_swap(p1, q1, false, false);
        const int q = 4 * f + 2 * p + h;
        *(uint4*)(row + (q ^ sw) * 16) = make_uint4(x[0], y[0], x[1], y[1]);
      }
    }
  }
  wave_lds_sync();
}

// Row pieces of one staged round (RB bytes per row, 16 bytes per lane): store
// k covers rows RPI k .. RPI k + RPI - 1.
template <int OSZ, int FBR>
struct RestRound {
  static constexpr int RB = FBR * 32 * OSZ;   // bytes per row piece (128 or 256)
  static constexpr int LPR = RB / 16;         // lanes per row piece
  static constexpr int RPI = 64 / LPR;        // rows per store instruction
  static constexpr int NST = kDecTok / RPI;   // store instructions
  static constexpr int K1 = NST / 4 - 1, K2 = 3 * NST / 4 - 1;   // fill points
  static_assert(K1 >= 0 && K1 < K2, "a round has at least four stores");
  static_assert(RB <= kRestStgRow && LPR >= 8, "a staged row fits and holds 8 swizzled chunks");
};

// Store k of a staged round, in two parts: rest_load reads the lane's 16
// bytes and output row from LDS (issued ahead of the store, so the store does
// not wait on LDS behind other waves' traffic), rest_put issues the 16-byte
// store to the row piece's output row, or to the sink when the row has no
// destination, and returns whether the row's block table entry was bad.
template <int OSZ, int FBR>
__device__ __forceinline__ void rest_load(int k, const uint8_t* stg, const int* rows, uint4& v, int& row) {
  using R = RestRound<OSZ, FBR>;
  const int lane = threadIdx.x & 63;
  const int c = lane % R::LPR;
  const int r = k * R::RPI + lane / R::LPR;
  v = *(const uint4*)(stg + r * R::RB + ((c ^ (r & 7)) * 16));
  row = rows[r];
}
template <int OSZ, int FBR>
__device__ __forceinline__ bool rest_put(const uint4& v, int row, uint8_t* dst_w, uint8_t* sink, bool store_ok,
                                         int F, int fb0, uint32_t row_lim) {
  using R = RestRound<OSZ, FBR>;
  const int lane = threadIdx.x & 63;
  const int col = (lane % R::LPR) * 16;
  uint8_t* p = store_ok && row >= 0 && (uint32_t)row < row_lim ? dst_w + ((size_t)row * F + 32 * fb0) * OSZ + col
                                                               : sink + (lane & 15) * 16;
  // non-temporal stores: the output streams to memory without leaving dirty
  // lines in the caches (plain stores measured faster for this kernel alone,
  // but the next kernel then pays for writing those lines back)
  __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), (u32x4*)p);
  return row == -2;
}

// Stores whose LDS reads are in flight ahead of the store being issued.
constexpr int kRestPrefetch = 8;

template <int KS, int NFB, bool FUSED, bool OUT32, bool PC>
__global__ __launch_bounds__(kRestThreads) __attribute__((amdgpu_waves_per_eu(2))) void restore_kernel(const LaunchArgs a) {
  static_assert(FUSED || !PC, "stage 2 reads the staging, whatever the record layout");
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ int pflag;
  constexpr int FPW = 32 * NFB;                 // features per wave
  constexpr int SLAB = rest_slab(NFB);
  constexpr int KA = KS > 0 ? KS : 1;
  constexpr size_t FB = rest_frag_bytes(KS);
  constexpr int OSZ = OUT32 ? 4 : 2;
  constexpr int FBR = OUT32 ? 2 : NFB;          // feature blocks per staged round
  constexpr int NRD = NFB / FBR;                // rounds per unit (1, or 2 for f32 at nfb 4)
  using R = RestRound<OSZ, FBR>;
  // 16-byte vectors per thread: a block's records (rb <= 24 KS) or staging
  constexpr int NVR = FUSED ? (kDecTok * 24 * KS / 16 + kRestThreads - 1) / kRestThreads : 0;
  constexpr int NVS = FUSED ? 0 : (KS > 0 ? ((int)stg_block_bytes(KS) / 16 + kRestThreads - 1) / kRestThreads : 0);
  constexpr int NXV = NVR > NVS ? NVR : (NVS > 0 ? NVS : 1);
  constexpr int NMU = (SLAB + kRestThreads - 1) / kRestThreads;   // mu values per thread
  constexpr int NSTORES = NRD * R::NST;         // store instructions per unit and wave
  static_assert(SLAB * 4 <= (int)kRestMuBytes, "a slab's mu fits its LDS buffer");
  const int F = a.F;
  const int tid = threadIdx.x;
  const int lane = tid & 63, t = lane & 31, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t g = logical_tile(), ng = gridDim.x;
  const int in_esz = a.dtype == KVTC_F32 ? 4 : 2;
  const uint32_t n_slabs = (uint32_t)((F + SLAB - 1) / SLAB);

  uint8_t* const stg = smem + kRestStgOff + (size_t)wave * kDecTok * kRestStgRow;
  uint8_t* const frag0 = smem + kRestFragOff;
  uint8_t* const rec0 = smem + kRestFragOff + 3 * FB;
  const uint32_t rec_lds = a.wave_lds;
  const size_t rec_rows_off = rec_lds - kDecTok * 4;
  auto recb = [&](uint32_t u) { return rec0 + (u & 1u) * rec_lds; };

  const uint32_t U = a.total_tiles;
  const uint32_t u_lo = (uint32_t)((uint64_t)U * g / ng), u_hi = (uint32_t)((uint64_t)U * (g + 1) / ng);

  if (u_lo < u_hi) {   // uniform: the workgroup has units
    // ---- loads of a unit into registers, and their commit to LDS. The
    // per-job fields are kept while consecutive units share the job.
    struct Src {
      int j;
      const uint8_t* base;   // FUSED: the job's records; else: its staging
      const uint8_t* hdr;    // the stream (its header is always readable)
      uint32_t rb, rbp, mrb;
    };
    auto src_of = [&](int j) __attribute__((always_inline)) {
      Src q;
      const JobDesc& jd = a.jobs[j];
      q.j = j;
      q.hdr = (const uint8_t*)jd.src;
      if (FUSED) {
        CSlot& sl = slot_of(a, jd.slot);
        q.rb = (uint32_t)sl.record_bytes;
        q.rbp = (uint32_t)dec_rec_stride((int)q.rb);
        // row of record byte x: (x * mrb) >> 24 = x / rb exactly for x < 2^24 / rb
        q.mrb = q.rb ? (0xFFFFFFu + q.rb) / q.rb : 0u;
        q.base = q.hdr + record_base(jd, F, in_esz);
      } else {
        q.rb = q.rbp = q.mrb = 0;
        q.base = (const uint8_t*)jd.staging;
      }
      return q;
    };
    auto fetch = [&](const RUnit& r, const Src& q, u32x4 (&xv)[NXV], int& ent, int& in) __attribute__((always_inline)) {
      const JobDesc& jd = a.jobs[r.j];
      if (FUSED) {
        const uint8_t* src = q.base + (size_t)r.c * kDecTok * q.rb;
        const uint32_t nbytes = r.nrec * q.rb, nvv = nbytes / 16u;
#pragma unroll
        for (int i = 0; i < NVR; ++i) {
          const uint32_t v = (uint32_t)(tid + kRestThreads * i);
          // vector nvv (a ragged end): the 16 bytes that end at the block's
          // last byte (at least 48 bytes into the stream, so in bounds); past
          // the block: the stream header
          const uint8_t* pv = v < nvv ? src + (size_t)v * 16
                            : v == nvv && nbytes > nvv * 16u ? src + nbytes - 16 : q.hdr;
          xv[i] = *(const u32x4*)pv;
        }
      } else {
        const uint8_t* blk = q.base + (size_t)r.c * stg_block_bytes(KS);
        constexpr uint32_t nv = (uint32_t)stg_block_bytes(KS) / 16u;
#pragma unroll
        for (int i = 0; i < NVS; ++i) {
          const uint32_t v = (uint32_t)(tid + kRestThreads * i);
          xv[i] = *(const u32x4*)(blk + (size_t)(v < nv ? v : 0u) * 16);
        }
      }
      in = rest_row_entry(jd, r.c, tid, ent);
    };
    auto commit = [&](const RUnit& r, const Src& q, const u32x4 (&xv)[NXV], int ent, int in, uint8_t* dstb,
                      int* rows) __attribute__((always_inline)) {
      const JobDesc& jd = a.jobs[r.j];
      if (FUSED) {
        const uint32_t nbytes = r.nrec * q.rb, nvv = nbytes / 16u;
#pragma unroll
        for (int i = 0; i < NVR; ++i) {
          const uint32_t v = (uint32_t)(tid + kRestThreads * i);
          const uint32_t x = v * 16u;
          // byte x goes to x + (x / rb) (rbp - rb); a vector never straddles rows
          if (v < nvv) {
            *(u32x4*)(dstb + x + ((x * q.mrb) >> 24) * (q.rbp - q.rb)) = xv[i];
          } else if (v == nvv && nbytes > x) {
            // the ragged end (then rb % 16 != 0 and rbp == rb): bytes
            // [x, nbytes) are the last nbytes - x of the vector
            const uint32_t o = 16u - (nbytes - x);
#pragma unroll
            for (uint32_t b = 0; b < 16; ++b)
              if (b >= o) dstb[nbytes - 16u + b] = (uint8_t)(xv[i][b / 4] >> (8 * (b % 4)));
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < NVS; ++i) {
          const uint32_t v = (uint32_t)(tid + kRestThreads * i);
          if (v < (uint32_t)stg_block_bytes(KS) / 16u) *(u32x4*)(dstb + (size_t)v * 16) = xv[i];
        }
      }
      if (tid < kDecTok) rows[tid] = rest_row(jd, r.c, tid, in, ent);
    };

    // ---- FUSED: B fragments and token scales of a unit from its records
    // (the arithmetic of stage 1), one K step per wave. The job's record
    // layout and this wave's group widths are kept in scalars while
    // consecutive units share the job, so a build issues no dependent loads
    // of them.
    constexpr int NSW = (KS + kRestWaves - 1) / kRestWaves;   // K steps per wave
    struct BuildJob {
      int j, rbp, G, n_g;
      int w[NSW > 0 ? NSW : 1], chunk[NSW > 0 ? NSW : 1];
      const uint32_t* pcw;   // PC: the slot's (record bit << 8) | width per component
    };
    auto build_job = [&](int j) __attribute__((always_inline)) {
      BuildJob bj;
      const JobDesc& jd = a.jobs[j];
      CSlot& sl = slot_of(a, jd.slot);
      bj.j = j;
      bj.rbp = dec_rec_stride(sl.record_bytes);
      bj.G = sl.G;
      bj.n_g = 16 * KS / bj.G;
      bj.pcw = PC ? (const uint32_t*)(a.state + sl.pcw_off) : nullptr;
#pragma unroll
      for (int i = 0; i < NSW; ++i) {
        const int s = wave + kRestWaves * i;
        const int ag = s < KS ? 16 * s / bj.G : 0;
        bj.w[i] = slot_width(sl, ag);
        bj.chunk[i] = slot_chunk(sl, ag);
      }
      return bj;
    };
    auto build = [&](const RUnit& r, const BuildJob& bj, const uint8_t* recs, uint8_t* fr)
        __attribute__((always_inline)) {
      const bool tok_ok = (uint32_t)t < r.nrec;
      const uint8_t* rr = recs + (tok_ok ? t : 0) * bj.rbp;
#pragma unroll
      for (int i = 0; i < NSW; ++i) {
        const int s = wave + kRestWaves * i;
        if (s < KS) {   // uniform per wave
          // S_t from every active group of the token (the K steps cover
          // 16 KS / G of them): lane half h takes groups h, h + 2, ..., and
          // the halves combine (permlane32 swap: each lane sees both)
          float m = 0.f;
#pragma unroll 4
          for (int a2 = h; a2 < bj.n_g; a2 += 2) {
            const float2 ps = get_scales(rr, a2);
            m = fmaxf(m, fmaxf(fabsf(ps.x), fabsf(ps.x + ps.y)));
          }
          {
            const auto mm = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
            m = fmaxf(__uint_as_float(mm[0]), __uint_as_float(mm[1]));
          }
          float S, Sinv;
          token_scale(m, S, Sinv);
          const int ag = 16 * s / bj.G;
          const float2 ps = get_scales(rr, ag);
          uint4 f = make_uint4(0u, 0u, 0u, 0u);
          if constexpr (PC) {
            if (tok_ok) f = frag_pc(rr, bj.pcw + 16 * s + 8 * h, ps.x, ps.y, Sinv);
          } else {
            const int w = bj.w[i];
            const float kf = (float)((1 << w) - 1);
            const uint64_t bits = lds_u64(rr + bj.chunk[i] + ((16 * s + 8 * h - ag * bj.G) * w) / 8);
            if (tok_ok) f = frag_from_bits(bits, ps.x, ps.y, w, kf, 1.0f / kf, Sinv);
          }
          *(uint4*)(fr + s * 1024 + lane * 16) = f;
          if (s == 0 && h == 0) *(float*)(fr + KS * 1024 + t * 4) = tok_ok ? S : 1.f;
        }
      }
      if (wave == kRestWaves - 1 && lane < kDecTok)   // the block's output rows
        ((int*)(fr + stg_block_bytes(KS)))[lane] = ((const int*)(recs + rec_rows_off))[lane];
    };

    // ---- the (job, slab) segment whose V' fragments and mu are loaded:
    // seg_issue issues the loads, seg_finish consumes them. The mu of two
    // segments is kept (by parity), since a unit is stored during the next
    // unit's iteration, which may start a segment.
    int seg_j = -1;
    uint32_t seg_slab = 0, seg_par = 1;
    bool job_ok = false;
    uint4 A[NFB][KA];
    float mreg[NMU];
    int f_w = 0;          // first feature of this wave
    bool active = false;  // the wave has features (f_w < F)
    auto mu_buf = [&](uint32_t par) { return (float*)(smem + kRestMuOff + par * kRestMuBytes); };
    auto seg_issue = [&](const RUnit& r) __attribute__((always_inline)) {
      seg_j = r.j;
      seg_slab = r.slab;
      seg_par ^= 1u;
      const JobDesc& jd = a.jobs[r.j];
      CSlot& sl = slot_of(a, jd.slot);
      const int f0 = (int)r.slab * SLAB;
      const float* mu = (const float*)(a.state + sl.mu_off);
#pragma unroll
      for (int i = 0; i < NMU; ++i) {
        const int fi = f0 + tid + kRestThreads * i;
        mreg[i] = mu[fi < F ? fi : 0];
      }
      f_w = f0 + wave * FPW;
      active = f_w < F;
      if (active) {
        // one coalesced 1 KB load per operand (the state stores V' in
        // operand order)
        const uint8_t* vdec = a.state + sl.vdec_off;
        const int nks = sl.r_dec >> 4;
#pragma unroll
        for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
          for (int s = 0; s < KS; ++s)
            A[fb][s] = *(const uint4*)(vdec + (((size_t)((f_w >> 5) + fb) * nks + s) * 64 + lane) * 16);
      }
      job_ok = FUSED ? check_header(a, jd, sl) == KVTC_OK : prior_rank(a, jd.status_idx) == 0;
    };
    auto seg_finish = [&]() __attribute__((always_inline)) {
      float* mu_s = mu_buf(seg_par);
#pragma unroll
      for (int i = 0; i < NMU; ++i) {
        const int li = tid + kRestThreads * i;
        if (li < SLAB) mu_s[li] = seg_slab * SLAB + li < (uint32_t)F ? mreg[i] : 0.f;
      }
      // the segment's loads (the V' fragments too) complete here, on every
      // path: no register enters the unit loop awaiting a load
      wait_vmcnt<0>();
    };

    // ---- the unit whose product is in acc and is stored during the next
    // iteration (p_real false before the first unit: its stores go to the
    // sink)
    f32x16 acc[NFB];
#pragma unroll
    for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[fb][i] = 0.f;
    bool p_real = false, p_ok = false;
    int p_j = 0, p_fw = 0;
    uint32_t p_par = 0, p_fi = 0;
    // Jobs (bit j) with a bad block table entry among the stored rows,
    // reported after the loop: a status atomic among the loop's loads and
    // stores would make the compiler treat the memory counter as out of
    // order and drain every store before each wait for a load.
    uint32_t bad_jobs = 0;

    auto fragb = [&](uint32_t fi) { return frag0 + fi * FB; };
    // The stores of the pending unit, with mfma(i) (K step i of this unit)
    // and fill() (the next unit's fragments) spread between them. Every wave
    // issues the same stores on every path (addresses are clamped or sent to
    // the sink), so the compiler can count them.
    auto store_pending = [&](auto&& mfma, auto&& fill) __attribute__((always_inline)) {
      const uint8_t* pf = fragb(p_fi);
      const float S = KS > 0 ? *(const float*)(pf + KS * 1024 + t * 4) : 1.f;
      const int* rows = (const int*)(pf + stg_block_bytes(KS));
      const float* mu_w = mu_buf(p_par) + (p_fw - (p_fw / SLAB) * SLAB);
      const JobDesc& jd = a.jobs[p_j];
      uint8_t* dst_w = (uint8_t*)jd.dst + (size_t)p_fw * OSZ;
      const bool store_ok = p_real && p_ok && p_fw < F;
      const uint32_t row_lim = rest_row_limit(jd);
      // the waves that fill in early are one per SIMD (waves go to the SIMDs
      // round robin), so every SIMD keeps a wave issuing stores
      const bool early = wave < 4;
      bool bad = false;
      static_for<NRD>([&](auto rdc) __attribute__((always_inline)) {
        constexpr int rd = decltype(rdc)::value;
        rest_stage<OSZ, FBR, NFB>(acc, rd * FBR, S, mu_w, stg);
        if constexpr (rd == NRD - 1) {
          // acc is free: this unit's product starts from zero
#pragma unroll
          for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[fb][i] = 0.f;
        }
        // slot i: the stores k with k KA / NST == i (spread over the K
        // steps), then, in the last round, K step i of this unit. The LDS
        // reads of store k are issued PFD stores ahead.
        constexpr int NSLOT = R::NST > KA ? R::NST : KA;
        constexpr int PFD = kRestPrefetch < R::NST ? kRestPrefetch : R::NST;
        uint4 sv[R::NST];
        int srow[R::NST];
        static_for<PFD>([&](auto kc) __attribute__((always_inline)) {
          constexpr int k = decltype(kc)::value;
          rest_load<OSZ, FBR>(k, stg, rows, sv[k], srow[k]);
        });
        static_for<NSLOT>([&](auto ic) __attribute__((always_inline)) {
          constexpr int i = decltype(ic)::value;
          __builtin_amdgcn_sched_barrier(0);
          static_for<R::NST>([&](auto kc) __attribute__((always_inline)) {
            constexpr int k = decltype(kc)::value;
            if constexpr (k * KA / R::NST == i) {
              if constexpr (k + PFD < R::NST) rest_load<OSZ, FBR>(k + PFD, stg, rows, sv[k + PFD], srow[k + PFD]);
              bad |= rest_put<OSZ, FBR>(sv[k], srow[k], dst_w, a.sink, store_ok, F, rd * FBR, row_lim);
              if constexpr (rd == 0 && (k == R::K1 || k == R::K2)) {
                if (early == (k == R::K1)) {   // uniform
                  __builtin_amdgcn_sched_barrier(0);
                  fill();
                  __builtin_amdgcn_sched_barrier(0);
                }
              }
            }
          });
          if constexpr (rd == NRD - 1 && i < KS) mfma(ic);
        });
        __builtin_amdgcn_sched_barrier(0);
        wave_lds_sync();   // the staging rows are free for the next round
      });
      if (p_real && __builtin_amdgcn_ballot_w64(bad) != 0) bad_jobs |= 1u << p_j;
    };

    // ---- prologue: the first units' loads and the first segment's loads
    // are all issued before any is waited for
    RUnit cur = rest_unit_at(a, u_lo, u_hi);
    RUnit nx = rest_next(a, cur, n_slabs);
    Src sq = src_of(cur.j);                 // the job of the unit last fetched
    u32x4 xv[NXV], xv2[NXV];
    int ent, in, ent2 = 0, in2 = 0;
    // fragment buffers (0..2, rotating): of the pending unit, of this unit,
    // of the next one
    uint32_t fi_cur = 0, fi_nx = 1;
    p_fi = 2;
    fetch(cur, sq, xv, ent, in);
    const Src sq2 = FUSED && nx.j >= 0 ? src_of(nx.j) : sq;
    if (FUSED) fetch(nx.j >= 0 ? nx : cur, sq2, xv2, ent2, in2);
    seg_issue(cur);
    if (FUSED) {
      commit(cur, sq, xv, ent, in, recb(u_lo), (int*)(recb(u_lo) + rec_rows_off));
      commit(nx.j >= 0 ? nx : cur, sq2, xv2, ent2, in2, recb(u_lo + 1), (int*)(recb(u_lo + 1) + rec_rows_off));
    } else {
      commit(cur, sq, xv, ent, in, fragb(fi_cur), (int*)(fragb(fi_cur) + stg_block_bytes(KS)));
    }
    seg_finish();
    __syncthreads();
    BuildJob bjob = build_job(cur.j);
    if (FUSED) {
      sq = sq2;
      build(cur, bjob, recb(u_lo), fragb(fi_cur));
      __syncthreads();
    }
    // Every load of the prologue has completed, also in lanes that had no use
    // for theirs: the loop starts with no register awaiting a load, so the
    // compiler needs no wait for the loop's stores before reusing registers.
    wait_vmcnt<0>();

    for (uint32_t u = u_lo; u < u_hi; ++u) {
      if (cur.j != seg_j || cur.slab != seg_slab) {   // uniform: a new segment
        seg_issue(cur);
        seg_finish();
        __syncthreads();
      }
      const RUnit nx_old = nx;
      // B fragments of this unit, K step s, from LDS into the MFMAs
      const uint8_t* fr = fragb(fi_cur);
      const bool act = active;
      auto mfma = [&](auto sc) __attribute__((always_inline)) {
        constexpr int s = decltype(sc)::value;
        if (act) {
          const f16x8 b = __builtin_bit_cast(f16x8, *(const uint4*)(fr + s * 1024 + lane * 16));
#pragma unroll
          for (int fb = 0; fb < NFB; ++fb)
            acc[fb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, A[fb][s]), b, acc[fb], 0, 0, 0);
        }
      };
      // Every iteration issues the same loads and commits them (past the
      // range the current unit is loaded again into a buffer nothing reads),
      // so the compiler can count the stores between the loads and the wait
      // for them.
      if (FUSED) {
        const RUnit nx2 = rest_next(a, nx, n_slabs);
        const RUnit fu = nx2.j >= 0 ? nx2 : cur;
        if (nx.j >= 0 && nx.j != bjob.j) bjob = build_job(nx.j);   // uniform
        if (fu.j != sq.j) sq = src_of(fu.j);
        fetch(fu, sq, xv, ent, in);
        __builtin_amdgcn_sched_barrier(0);
        // the previous unit is stored while this one is multiplied and the
        // next one dequantized
        store_pending(mfma, [&] {
          if (nx.j >= 0) build(nx, bjob, recb(u + 1), fragb(fi_nx));
        });
        __builtin_amdgcn_sched_barrier(0);
        commit(fu, sq, xv, ent, in, recb(u), (int*)(recb(u) + rec_rows_off));
        nx = nx2;
      } else {
        const RUnit fu = nx.j >= 0 ? nx : cur;
        if (fu.j != sq.j) sq = src_of(fu.j);
        fetch(fu, sq, xv, ent, in);
        __builtin_amdgcn_sched_barrier(0);
        store_pending(mfma, [] {});
        __builtin_amdgcn_sched_barrier(0);
        commit(fu, sq, xv, ent, in, fragb(fi_nx), (int*)(fragb(fi_nx) + stg_block_bytes(KS)));
        nx = rest_next(a, nx, n_slabs);
      }
      // the loads of this iteration have completed (only its stores may be
      // outstanding), on every path through commit
      wait_vmcnt<NSTORES>();
      __syncthreads();
      // this unit becomes the pending one
      p_real = true;
      p_ok = job_ok;
      p_j = cur.j;
      p_fw = f_w;
      p_par = seg_par;
      const uint32_t fi_free = p_fi;
      p_fi = fi_cur;
      fi_cur = fi_nx;
      fi_nx = fi_free;
      cur = nx_old;
    }
    // the last unit
    store_pending([](auto) {}, [] {});
    // reported once every store is issued
    if (tid % 64 == 0) {
      for (uint32_t m = bad_jobs; m; m &= m - 1) set_status(a, a.jobs[__builtin_ctz(m)].status_idx, KVTC_E_INVALID);
    }
  }

  if (FUSED) {
    // Header and passthrough units (kRestPassRows rows each; job j owns
    // max(1, units) of them from cblk_begin, its first one records the header
    // check in the job's status word), split evenly over the workgroups; run
    // last, while the last unit's stores drain. (The compressed rows check
    // the header themselves.)
    const uint32_t P = a.total_cblks;
    const uint32_t p_end = (uint32_t)((uint64_t)P * (g + 1) / ng);
    const uint32_t p_lo = (uint32_t)((uint64_t)P * g / ng);
    int j = p_lo < p_end ? job_at<&JobDesc::cblk_begin>(a, p_lo) : 0;
    __syncthreads();   // the passthrough row list reuses LDS
    for (uint32_t p = p_lo; p < p_end; ++p) {
      while (j + 1 < a.n_jobs && a.jobs[j + 1].cblk_begin <= p) ++j;   // usually no step
      const JobDesc& jd = a.jobs[j];
      const uint32_t lp = p - jd.cblk_begin;
      const int st = check_header(a, jd, slot_of(a, jd.slot));   // uniform
      if (lp == 0 && tid == 0) set_status(a, jd.status_idx, st);
      if (st != KVTC_OK) continue;
      if (tid == 0) pflag = 0;
      __syncthreads();
      bool ok = true;
      if (lp * kRestPassRows < jd.s1 + jd.w1)
        ok = decode_passthrough<kRestThreads, kRestPassRows>(a, jd, lp, (long*)smem);
      if (!ok) atomicExch(&pflag, 1);
      __syncthreads();
      if (tid == 0 && pflag) set_status(a, jd.status_idx, KVTC_E_INVALID);
      __syncthreads();   // row list and flag are free for the next unit
    }
  }
}

// Test hook: records -> codes (u8, one per component) and (shift, scale)
// pairs, through the decode's record readers (code_bits8, codes8_w,
// get_scales).
template <int G>
__global__ __launch_bounds__(kThreads) void unpack_kernel(const LaunchArgs a, uint8_t* codes, float2* ssg) {
  extern __shared__ __align__(16) uint8_t smem[];
  const uint32_t tile = logical_tile();
  if (tile >= a.total_tiles) return;
  const JobDesc& jd = a.jobs[0];
  CSlot& sl = slot_of(a, jd.slot);
  const uint32_t lt = tile - jd.tile_begin;
  if (lt >= jd.n_ctiles || sl.r_eff == 0) return;
  const uint32_t t0 = lt * kUnpackTile;
  const uint32_t n = min((uint32_t)kUnpackTile, jd.tc - t0);
  const int esz = a.dtype == KVTC_F32 ? 4 : 2;
  const int rb = sl.record_bytes;
  const uint8_t* recs = (const uint8_t*)jd.src + record_base(jd, a.F, esz) + (size_t)t0 * rb;
  stage_to_lds(smem, recs, (size_t)n * rb);
  __syncthreads();
  // One thread per (token, 8-component chunk).
  const int chunks = sl.r_eff / 8;
  for (int idx = threadIdx.x; idx < (int)n * chunks; idx += kThreads) {
    const int tl = idx / chunks, c = (idx % chunks) * 8;
    const uint8_t* rec = smem + (size_t)tl * rb;
    const int ag = c / G, o = c % G;
    const int w = slot_width(sl, ag);
    uint32_t v[8];
    codes8(code_bits8(rec, sl, ag, o, w), w, v);
    uint64_t out = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) out |= (uint64_t)v[j] << (8 * j);
    *(uint64_t*)(codes + (size_t)(t0 + tl) * sl.r_eff + c) = out;
    if (o == 0) ssg[(size_t)(t0 + tl) * sl.n_act + ag] = get_scales(rec, ag);
  }
}


// ------------------------------------------------------------- launchers ---

#define KVTC_KS_CASES(X)                                                          \
  X(0) X(1) X(2) X(3) X(4) X(5) X(6) X(7) X(8) X(9) X(10) X(11) X(12) X(13) X(14) \
  X(15) X(16)

int launch_prep(const LaunchArgs& a, int ks, size_t lds, hipStream_t s) {
  // one wave per compressed block; any grid covers the passthrough units
  const dim3 g = grid_for(std::max(8u, (a.total_tiles + kWaves - 1) / kWaves));
#define KVTC_PREP(KV)                                                             \
  case KV:                                                                        \
    if (a.pc) {                                                                   \
      allow_lds(prep_kernel<KV, true>, lds);                                      \
      hipLaunchKernelGGL((prep_kernel<KV, true>), g, dim3(kThreads), lds, s, a);  \
    } else {                                                                      \
      allow_lds(prep_kernel<KV, false>, lds);                                     \
      hipLaunchKernelGGL((prep_kernel<KV, false>), g, dim3(kThreads), lds, s, a); \
    }                                                                             \
    break;
  switch (ks) {
    KVTC_KS_CASES(KVTC_PREP)
    default:
      return (int)hipErrorInvalidValue;
  }
#undef KVTC_PREP
  return (int)hipGetLastError();
}

// Restore launch: nfb from the K-step count and F; at most 8 / kRestWaves
// workgroups per CU (the occupancy query), fewer when there are few units.
template <bool FU, bool O32, bool PC>
static int launch_restore_t(const LaunchArgs& a, int ks, size_t lds, hipStream_t s) {
  const int nfb = rest_nfb(ks, a.F);
#define KVTC_REST(KV, NFBV)                                                                      \
  if (ks == KV && nfb == NFBV) {                                                                 \
    allow_lds(restore_kernel<KV, NFBV, FU, O32, PC>, lds);                                           \
    const dim3 g(std::min({std::max(8u, (a.total_tiles + 7u) / 8u * 8u),                         \
                           resident_grid(restore_kernel<KV, NFBV, FU, O32, PC>, kRestThreads, lds,  \
                                         8 / kRestWaves),                                        \
                           persistent_grid_cap()}));                                             \
    hipLaunchKernelGGL((restore_kernel<KV, NFBV, FU, O32, PC>), g, dim3(kRestThreads), lds, s, a);  \
    return (int)hipGetLastError();                                                               \
  }
#define KVTC_REST4(KV) KVTC_REST(KV, 4)
#define KVTC_REST2(KV) KVTC_REST(KV, 2)
  KVTC_REST4(0) KVTC_REST4(1) KVTC_REST4(2) KVTC_REST4(3) KVTC_REST4(4) KVTC_REST4(5) KVTC_REST4(6)
  KVTC_KS_CASES(KVTC_REST2)
#undef KVTC_REST2
#undef KVTC_REST4
#undef KVTC_REST
  return (int)hipErrorInvalidValue;
}

int launch_restore(const LaunchArgs& a, int ks, bool fused, size_t lds, hipStream_t s) {
  const bool o32 = a.out_dtype == KVTC_F32;
  if (fused && a.pc)   // the fused build reads each code at its own bit and width
    return o32 ? launch_restore_t<true, true, true>(a, ks, lds, s) : launch_restore_t<true, false, true>(a, ks, lds, s);
  return fused ? (o32 ? launch_restore_t<true, true, false>(a, ks, lds, s)
                      : launch_restore_t<true, false, false>(a, ks, lds, s))
               : (o32 ? launch_restore_t<false, true, false>(a, ks, lds, s)
                      : launch_restore_t<false, false, false>(a, ks, lds, s));
}

int launch_unpack(const LaunchArgs& a, int G, size_t lds, void* codes, void* ss, hipStream_t s) {
  const dim3 g = grid_for(a.total_tiles);
  if (G == 16) {
    allow_lds(unpack_kernel<16>, lds);
    hipLaunchKernelGGL((unpack_kernel<16>), g, dim3(kThreads), lds, s, a, (uint8_t*)codes, (float2*)ss);
  } else if (G == 32) {
    allow_lds(unpack_kernel<32>, lds);
    hipLaunchKernelGGL((unpack_kernel<32>), g, dim3(kThreads), lds, s, a, (uint8_t*)codes, (float2*)ss);
  } else {
    return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

// ----------------------------------------------- decode without allocation ---
//
// Status words and sink of kvtc_decode_noalloc: a workspace of
// kvtc_workspace_bytes(kMaxScratchJobs) bytes in a static device array (one
// copy per GPU, held until the process ends). Host code never passes the
// array's name to a kernel (on the host it is only a stand-in): each device's
// address comes from hipGetSymbolAddress, once, with that device current.
constexpr int kMaxScratchJobs = KVTC_MAX_JOBS;
constexpr size_t kScratchBytes = ((size_t)kMaxScratchJobs * 8 + 255) / 256 * 256 + kSinkBytes;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // per device, null until looked up
}  // namespace

int noalloc_scratch(void** ptr, size_t* bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    if (!p) return (int)hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  *bytes = kScratchBytes;
  return (int)hipSuccess;
}

// Zero n status words (a fill kernel, not a memset node, so the call can sit
// in a captured graph and be replayed).
__global__ void clear_words_kernel(unsigned long long* w, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) w[i] = 0ull;
}
// Status words -> kvtc_status codes (the rank in the low byte).
__global__ void status_codes_kernel(const unsigned long long* w, int32_t* out, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = rank_status((int)(w[i] & 0xFFull));
}

int launch_clear_words(void* words, int n, hipStream_t s) {
  hipLaunchKernelGGL(clear_words_kernel, dim3((n + 255) / 256), dim3(256), 0, s, (unsigned long long*)words, n);
  return (int)hipGetLastError();
}
int launch_status_codes(const void* words, int32_t* out, int n, hipStream_t s) {
  hipLaunchKernelGGL(status_codes_kernel, dim3((n + 255) / 256), dim3(256), 0, s,
                     (const unsigned long long*)words, out, n);
  return (int)hipGetLastError();
}

}  // namespace kvtc
