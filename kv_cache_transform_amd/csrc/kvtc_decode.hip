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
// S_t * D + mu through LDS rows in 128-byte streaming stores.
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
template <int KS>
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
      int j = 0;
      for (int i = 1; i < a.n_jobs; ++i)
        if (a.jobs[i].cblk_begin <= p) j = i;
      const JobDesc& jd = a.jobs[j];
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
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const int ag = 16 * s / G;
    const int w = slot_width(sl, ag);
    const float kf = (float)((1 << w) - 1);
    const uint4 f = tok_ok ? frag_from_bits(code_bits8(r, sl, ag, 16 * s + 8 * h - ag * G, w), ps[s].x,
                                            ps[s].y, w, kf, 1.0f / kf, Sinv)
                           : make_uint4(0u, 0u, 0u, 0u);
    *(uint4*)(blk + s * 1024 + lane * 16) = f;
  }
  if (h == 0) *(float*)(blk + KS * 1024 + t * 4) = tok_ok ? S : 1.f;
}

// Stage 2 segment: features [f0, f0 + FS) x blocks [c_lo, c_hi) of kDecTok
// compressed tokens of one job. The slab of V' (fp16, FS rows of r_dec,
// padded by 16 bytes per row) and mu stay in LDS; each wave then runs on its
// own over every fourth block: it loads the block's B operands and
// scales (the next block's are in flight meanwhile), runs FS / 32 x KS
// MFMAs D[feature][token], forms S_t * D + mu and stores it through its LDS
// staging rows as 128-byte segments. Every store is issued (rows past the
// tile, or with a bad block table entry, go to the workspace sink), so the
// number of memory operations per block is fixed and the wait for the next
// block's operands never covers this block's stores.
template <int KS, bool OUT32>
__device__ void gemm_segment(const LaunchArgs& a, int j, uint32_t slab, uint32_t c_lo, uint32_t c_hi,
                             uint8_t* smem) {
  constexpr int FS = gemm_features(KS);
  constexpr int NFB = FS / 32;
  constexpr int OSZ = OUT32 ? 4 : 2;
  constexpr int BPS = 128 / (32 * OSZ);           // feature blocks per 128-byte segment
  constexpr int KA = KS > 0 ? KS : 1;
  constexpr int AST = KS * 32 + 16;               // LDS bytes per V' row
  const JobDesc& jd = a.jobs[j];
  CSlot& sl = slot_of(a, jd.slot);
  if (prior_rank(a, jd.status_idx) != 0) return;  // stage 1 rejected it
  const int F = a.F;
  const int f0 = (int)slab * FS;
  const uint32_t t0 = 0;
  const int lane = threadIdx.x & 63, h = lane >> 5, c16 = lane & 7;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));

  uint8_t* As = smem;
  float* mu_s = (float*)(smem + FS * AST);
  uint8_t* stg = smem + FS * AST + FS * 4 + wave * kDecTok * kOutRow;
  {
    const int r_dec = sl.r_dec;
    const uint8_t* vdec = a.state + sl.vdec_off;
    for (int i = threadIdx.x; i < FS * 2 * KS; i += kGemmThreads) {
      const int row = i / (2 * KS), c = i - row * (2 * KS);
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (f0 + row < F) v = *(const uint4*)(vdec + ((size_t)(f0 + row) * r_dec + 8 * c) * 2);
      *(uint4*)(As + row * AST + 16 * c) = v;
    }
    const float* mu = (const float*)(a.state + sl.mu_off);
    for (int i = threadIdx.x; i < FS; i += kGemmThreads) mu_s[i] = f0 + i < F ? mu[f0 + i] : 0.f;
  }
  __syncthreads();

  const uint8_t* stg_job = (const uint8_t*)jd.staging;
  constexpr size_t BB = stg_block_bytes(KS);
  const uint32_t tb0 = t0 / kDecTok;
  uint8_t* dst = (uint8_t*)jd.dst;
  uint8_t* sink = a.sink + c16 * 16;
  int bad = 0;
  // Job fields used per block, held in registers.
  const uint32_t tc = jd.tc, s1 = jd.s1;
  const int32_t* btab = jd.block_table;
  const int bsz = jd.block_size, bsh = jd.bs_shift, nblk = jd.n_blocks;

  // Operands of block c: B fragments, the lane's token scale and the block
  // table entries of the rows this lane stores (r = 8 it + lane / 8).
  uint4 Bn[KA];
  float Sn;
  int btn[4];
  auto fetch = [&](uint32_t c) {
    const uint8_t* blk = stg_job + (size_t)(tb0 + c) * BB;
#pragma unroll
    for (int s = 0; s < KS; ++s) Bn[s] = *(const uint4*)(blk + s * 1024 + lane * 16);
    // stage 1 writes no staging when no component is kept (KS == 0)
    Sn = KS > 0 ? *(const float*)(blk + KS * 1024 + (lane & 31) * 4) : 1.f;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const uint32_t tt = s1 + min(t0 + c * kDecTok + 8 * it + (lane >> 3), tc - 1);
      btn[it] = btab[bsh >= 0 ? tt >> bsh : tt / (uint32_t)bsz];
    }
  };
  // Operands in use: B fragments, token scale and the store addresses of
  // the lane's rows; taken over from the fetched ones only after the
  // block's stores were issued, so every wait covers loads alone.
  uint4 B[KA];
  float S;
  uint8_t* dp[4];
  auto take = [&](uint32_t c) {
#pragma unroll
    for (int s = 0; s < KS; ++s) B[s] = Bn[s];
    S = Sn;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const uint32_t tok = t0 + c * kDecTok + 8 * it + (lane >> 3);
      const uint32_t tt = s1 + tok;
      const int bt = btn[it];
      const bool blk_ok = bt >= 0 && bt < nblk;
      bad |= (int)(tok < tc && !blk_ok);
      const uint32_t in_blk = bsh >= 0 ? tt & ((1u << bsh) - 1u) : tt % (uint32_t)bsz;
      const long row = (long)bt * bsz + (long)in_blk;
      dp[it] = tok < tc && blk_ok ? dst + (row * F + f0) * OSZ + c16 * 16 : sink;
    }
  };
  if (c_lo + wave < c_hi) {
    fetch(c_lo + wave);
    take(c_lo + wave);
  }
  for (uint32_t c = c_lo + wave; c < c_hi; c += kGemmWaves) {
    fetch(min(c + kGemmWaves, c_hi - 1));   // unconditional: a fixed count of loads per block
    // Keep the scheduler from pulling the next block's takeover (which waits
    // for these loads) into this block's work.
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int fb = 0; fb < NFB; ++fb) {
      const uint8_t* arow = As + (fb * 32 + (lane & 31)) * AST + 16 * h;
      f32x16 acc;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
      for (int s = 0; s < KS; ++s)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, *(const uint4*)(arow + 32 * s)),
                                                     __builtin_bit_cast(f16x8, B[s]), acc, 0, 0, 0);
      // D[feature][token]: token lane % 32, features 8 qd + 4 h + {0..3}
      uint8_t* srow = stg + (lane & 31) * kOutRow + (fb % BPS) * 32 * OSZ;
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const int fl = 8 * qd + 4 * h;
        const float4 m4 = *(const float4*)(mu_s + 32 * fb + fl);
        const float o0 = __builtin_fmaf(acc[4 * qd + 0], S, m4.x);
        const float o1 = __builtin_fmaf(acc[4 * qd + 1], S, m4.y);
        const float o2 = __builtin_fmaf(acc[4 * qd + 2], S, m4.z);
        const float o3 = __builtin_fmaf(acc[4 * qd + 3], S, m4.w);
        if (OUT32)
          *(float4*)(srow + fl * 4) = make_float4(o0, o1, o2, o3);
        else
          *(uint2*)(srow + fl * 2) = make_uint2(pack_bf16x2(o0, o1), pack_bf16x2(o2, o3));
      }
      if (fb % BPS == BPS - 1) {
        const int fs = 32 * (fb - BPS + 1);            // segment's first feature in the slab
        const bool in_f = f0 + fs < F;                 // F % 64 == 0: whole segments
        wave_lds_sync();
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const uint4 v = *(const uint4*)(stg + (8 * it + (lane >> 3)) * kOutRow + c16 * 16);
          // streaming (non-temporal) stores: the output is not read back here
          __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v),
                                      (u32x4*)(dp[it] == sink || !in_f ? sink : dp[it] + fs * OSZ));
        }
        wave_lds_sync();
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    take(min(c + kGemmWaves, c_hi - 1));
  }
  if (bad) set_status(a, jd.status_idx, KVTC_E_INVALID);
  __syncthreads();  // the slab and staging rows are free for the next tile
}

// Stage 2 work is counted in units of one block of kDecTok tokens of one
// feature slab of one job, ordered (job, slab, block); job j's units start
// at tile_begin and number n_ctiles = slabs * blocks. The host launches at
// most as many workgroups as fit on the device at once and each takes an
// equal contiguous range of units, so all finish together; a range crosses
// few (job, slab) boundaries (the slab of V' is loaded once per segment),
// and the ranges in flight on one XCD cover the slabs of the same tokens.
template <int KS, bool OUT32>
__global__ __launch_bounds__(kGemmThreads) __attribute__((amdgpu_waves_per_eu(4))) void gemm_kernel(const LaunchArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const uint64_t U = a.total_tiles;
  const uint32_t g = logical_tile();
  uint32_t u = (uint32_t)(U * g / gridDim.x);
  const uint32_t u_end = (uint32_t)(U * (g + 1) / gridDim.x);
  while (u < u_end) {
    const int j = find_job(a, u);
    const JobDesc& jd = a.jobs[j];
    const uint32_t n_ch = (jd.tc + kDecTok - 1) / kDecTok;
    const uint32_t lu = u - jd.tile_begin;
    const uint32_t slab = lu / n_ch, c = lu - slab * n_ch;
    const uint32_t seg_end = min(u_end, jd.tile_begin + (slab + 1) * n_ch);
    gemm_segment<KS, OUT32>(a, j, slab, c, c + (seg_end - u), smem);
    u = seg_end;
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
#define KVTC_PREP(KV)                                                       \
  case KV:                                                                  \
    allow_lds(prep_kernel<KV>, lds);                                        \
    hipLaunchKernelGGL((prep_kernel<KV>), g, dim3(kThreads), lds, s, a);    \
    break;
  switch (ks) {
    KVTC_KS_CASES(KVTC_PREP)
    default:
      return (int)hipErrorInvalidValue;
  }
#undef KVTC_PREP
  return (int)hipGetLastError();
}

template <bool OUT32>
static int launch_gemm_o(const LaunchArgs& a, int ks, size_t lds, hipStream_t s) {
#define KVTC_GEMM(KV)                                                                        \
  case KV: {                                                                                 \
    allow_lds(gemm_kernel<KV, OUT32>, lds);                                                  \
    const dim3 g(std::min({std::max(8u, a.total_tiles / (8 * kGemmMinUnits) * 8),         \
                           resident_grid(gemm_kernel<KV, OUT32>, kGemmThreads, lds),       \
                           persistent_grid_cap()}));                                       \
    hipLaunchKernelGGL((gemm_kernel<KV, OUT32>), g, dim3(kGemmThreads), lds, s, a);              \
    break;                                                                                   \
  }
  switch (ks) {
    KVTC_KS_CASES(KVTC_GEMM)
    default:
      return (int)hipErrorInvalidValue;
  }
#undef KVTC_GEMM
  return (int)hipGetLastError();
}

int launch_gemm(const LaunchArgs& a, int ks, size_t lds, hipStream_t s) {
  return a.out_dtype == KVTC_F32 ? launch_gemm_o<true>(a, ks, lds, s) : launch_gemm_o<false>(a, ks, lds, s);
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

}  // namespace kvtc
