// HIP kernels of the compression side of KV-cache transform coding for
// gfx950 (MI355X): the encode and the kvtc_pack test hook.
//
// Method: "KV Cache Transform Coding for Compact Storage in LLM Inference"
// (gist.science, 2511.01815), section 2B: subtract the mean, multiply by V,
// quantize with the DP widths, pack.
//
// Encode (256 threads, persistent, at most two workgroups per CU): each wave
// owns 32 tokens of a tile. The projection runs on v_mfma_f32_32x32x16_bf16
// in transposed form, D[component][token] = sum_f V'^T[component][f] *
// d[token][f], where d is the token centred on the bf16 part of the mean and
// split into bf16 terms in registers as each B fragment is read. Token rows
// go through a per-wave LDS tile (row-contiguous loads), basis K-slices
// through two shared LDS buffers, both two slices ahead. In the accumulator
// layout a lane owns one token and half of every group's components, so the
// per-(token, group) min/max needs one cross-lane exchange (lane ^ 32) and
// quantization is lane-local; codes are OR-ed into LDS record rows and leave
// in 16-byte stores.
#include "kvtc_device.h"

namespace kvtc {

// --------------------------------------------------------------- encode ---

// Compressed rows carry their own index space of kEncBlk-token blocks
// (JobDesc::cblk_begin): the blocks of every job with records, job after job.
__device__ __forceinline__ int find_cblk_job(const LaunchArgs& a, uint32_t b) {
  return job_at<&JobDesc::cblk_begin>(a, b);
}
// The job of block b >= the first block of job j: j moved forward (a
// workgroup's blocks are contiguous, so this is usually zero or one step).
__device__ __forceinline__ int next_cblk_job(const LaunchArgs& a, int j, uint32_t b) {
  while (j + 1 < a.n_jobs && a.jobs[j + 1].cblk_begin <= b) ++j;
  return j;
}

// The value of lane l ^ 32 (the other half-wave), through
// v_permlane32_swap: with x in both operands the first result holds the low
// half in both halves, the second the high half in both.
__device__ __forceinline__ float xor32(float x, int h) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(h ? r[0] : r[1]);
}

// Quantize the projected tile held in acc (acc[b][i]: component
// 32b + 8(i/4) + 4h + i%4 of token tl) into the token's LDS record row rec,
// which the caller has zeroed. Lane h holds, of each group, the runs of four
// components 8m + 4h .. + 3 (m < G/8): their codes occupy bits
// [(8m + 4h) w, (8m + 4h + 4) w) of the group's chunk and are merged into
// the record with at most two 32-bit ORs per run (runs of the two lanes can
// share a word).
//
// With a width per component (sl.pc), component o of active group a is
// coded on its own 2^w - 1 levels of the group's range and ORed in at its
// own bit position; both come from the slot's table (pcw_off in state).
template <int NB, int G>
__device__ __forceinline__ void quantize_tile(const f32x16 (&acc)[NB], CSlot& sl, const uint8_t* state,
                                              uint8_t* rec, int h, bool tok_ok) {
  // A group of G components is the item range [(G/2) * sg, (G/2) * (sg + 1))
  // of block b with sg = a % (32/G).
  constexpr int SUB = 32 / G;
  uint32_t* const rw = (uint32_t*)rec;   // rec is 4-byte aligned (padded_stride)
#pragma unroll
  for (int b = 0; b < NB; ++b) {
#pragma unroll
    for (int sg = 0; sg < SUB; ++sg) {
      const int ag = b * SUB + sg;
      if (ag < sl.n_act) {
        float v[G / 2];
#pragma unroll
        for (int i = 0; i < G / 2; ++i) v[i] = acc[b][(G / 2) * sg + i];
        float mn = v[0], mx = v[0];
#pragma unroll
        for (int i = 1; i < G / 2; ++i) {
          mn = fminf(mn, v[i]);
          mx = fmaxf(mx, v[i]);
        }
        mn = fminf(mn, xor32(mn, h));
        mx = fmaxf(mx, xor32(mx, h));
        const float scale = mx - mn;
        if (sl.pc) {
          const uint32_t* pcw = (const uint32_t*)(state + sl.pcw_off) + ag * G;
#pragma unroll
          for (int m = 0; m < G / 8; ++m)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t ent = pcw[8 * m + 4 * h + e];
              const int wc = (int)(ent & 0xFFu);
              if (wc) {
                const float kc = (float)((1 << wc) - 1);
                const float invc = scale > 0.f ? kc / scale : 0.f;
                const float u = (v[4 * m + e] - mn) * invc;
                const float r = fminf(fmaxf(__builtin_rintf(u), 0.f), kc);
                if (tok_ok) or_code(rw, ent >> 8, (uint32_t)r, wc);
              }
            }
        } else {
          const int w = slot_width(sl, ag);
          const float k = (float)((1 << w) - 1);
          const float inv = scale > 0.f ? k / scale : 0.f;
#pragma unroll
          for (int m = 0; m < G / 8; ++m) {
            uint32_t run = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float d = v[4 * m + e] - mn;
              const float u = d * inv;
              const float r = fminf(fmaxf(__builtin_rintf(u), 0.f), k);
              run |= (uint32_t)r << (e * w);
            }
            if (tok_ok) or_code_run(rw, code_bit(sl, ag, 8 * m + 4 * h, w), run, w);
          }
        }
        if (tok_ok && h == 0) put_scales(rw, ag, mn, scale);
      }
      // One group at a time: interleaving them only raises register pressure.
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// Persistent encode. Each workgroup first writes the headers and passthrough
// units u = g, g + grid, ... of the launch, then projects, quantizes and
// packs an equal contiguous range of the compressed 32-token blocks, as
// tiles of up to four blocks of one job. Its four waves take a block of a
// tile each; the K loop walks slices of kEncKS features.
// The slice pipeline runs across tile boundaries: a load cursor two slices
// ahead of the computation moves on into the next tile of the range, so the
// loads of a tile's first slices are in flight during the previous tile's
// quantization, and the pipeline fills once per workgroup.
template <int NB, int G, bool F32IN, bool ODD, bool FOLD>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(!F32IN && NB <= 3 ? 2 : 1))) void encode_kernel(const LaunchArgs a) {
  static_assert(!(FOLD && F32IN), "only a bf16 token is an exact single MFMA operand");
  extern __shared__ __align__(16) uint8_t smem[];
  const uint32_t g = logical_tile();
  const int F = a.F;
  constexpr int esz = F32IN ? 4 : 2;
  const size_t row_bytes = (size_t)F * esz;
  for (uint32_t u = g; u < a.total_tiles; u += gridDim.x) {
    const JobDesc& jd = a.jobs[find_job(a, u)];
    const uint32_t lt = u - jd.tile_begin;
    if (lt == 0 && threadIdx.x == 0) {
      write_header(a, jd, slot_of(a, jd.slot));
      set_status(a, jd.status_idx, KVTC_OK);
    }
    if (lt >= jd.n_ctiles) encode_passthrough(jd, lt - jd.n_ctiles, row_bytes);
  }
  // This workgroup's blocks [b_begin, b_end), taken as tiles of up to
  // kEncWaves blocks of one job (tile_end); equal block counts per
  // workgroup keep them busy until the end of the launch.
  const uint32_t B = a.total_cblks;
  const uint32_t b_begin = (uint32_t)((uint64_t)B * g / gridDim.x);
  const uint32_t b_end = (uint32_t)((uint64_t)B * (g + 1) / gridDim.x);
  if (b_begin >= b_end) return;
  auto tile_end = [&](int j, uint32_t b) -> uint32_t {
    const JobDesc& jd = a.jobs[j];
    const uint32_t job_end = jd.cblk_begin + (jd.tc + kEncBlk - 1) / kEncBlk;
    return min(min(b + (uint32_t)kEncWaves, job_end), b_end);
  };

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5;
  const int tl = wave * 32 + (lane & 31);            // token within the tile
  static_assert(kEncWaves * 64 == kThreads, "one wave per 32 tokens of a tile");

  // LDS: two basis K-slices [32 * NB][kEncRowPad] bf16, the wave's token
  // tile (32 rows of the slice's raw input elements), then the centring
  // vector mu_hi (F fp32). Basis slices and token rows are
  // loaded from memory two slices ahead of their use: during slice i the
  // loads of slice i + 2 are issued, and at the end of slice i the token rows
  // of slice i + 1 go to the wave's token tiles and basis slice i + 1 to the
  // other basis buffer (last read in slice i - 1, before the barrier that
  // ended it). After a tile's last slice the records are assembled in LDS
  // from offset 0, then slice 0 of the next tile is staged. Loads past the
  // range's last slice re-read it, so every slice issues the same loads and
  // the waits count exactly.
  //
  // Centring (the mean is subtracted before the transform): each B fragment
  // is read raw from the token tile, centred on mu_hi = bf16_rne(mu32) in
  // fp32, d = x - mu_hi, and split into NT bf16 terms t_1 = bf16(d),
  // t_2 = bf16(d - t_1), ... in registers, right before its MFMAs (so this
  // arithmetic overlaps the previous K step's MFMAs); all terms are
  // multiplied, and the accumulators start at -(mu32 - mu_hi) V' (fp64, rounded
  // once, in the device state). For a bf16 token d is exact in fp32 and two
  // terms hold it exactly whenever x and mu_hi lie within a factor 2^8 of
  // each other (else to 2^-17 of |d|); for an f32 token d rounds once and
  // three terms hold it exactly. The product's rounding error therefore
  // scales with |x - mu| (the centred token), not with |x|: a mean large
  // against the spread costs no precision.
  //
  // Folded mean (FOLD, bf16 slots whose mean is no larger than their
  // spread): the stored bf16 token is the B fragment as it is (one term, no
  // centring arithmetic, no mean in LDS) and the accumulators start at
  // -mu32 V'. The error then scales with |x|, which such a mean keeps within
  // a factor of about sqrt(2) of |x - mu|.
  constexpr int NT = FOLD ? 1 : enc_terms(F32IN);
  constexpr int slice_elems = 32 * NB * kEncRowPad;
  constexpr int XROW = enc_xrow_bytes(F32IN);   // bytes per token tile row
  uint16_t* const vbase = (uint16_t*)smem;
  uint8_t* const xs = smem + 2 * enc_basis_bytes(NB) + wave * enc_xtile_bytes(F32IN);
  float* const mu_l = (float*)(smem + 2 * enc_basis_bytes(NB) + kEncWaves * enc_xtile_bytes(F32IN));
  const int n_sl = F / kEncKS;   // odd exactly when ODD (the host picks the kernel)

  // Load cursor: tile lc, slice lk; the tile's basis and token row offsets.
  // Rows past the tile's last token re-read its first row; their results
  // are dropped.
  constexpr int CH = kEncKS * esz / 16;   // 16-byte chunks per row segment
  constexpr int RPI = 64 / CH;            // rows per load instruction
  constexpr int NI = 32 / RPI;            // load instructions per slice
  constexpr int EPC = 16 / esz;           // features per chunk
  const int cx = lane % CH;
  uint32_t lbe;       // end block of the load cursor's tile
  int lk = 0;
  const int j_begin = find_cblk_job(a, b_begin);
  int lj = j_begin;   // the load cursor's job
  const uint16_t* l_venc;
  const uint8_t* l_x;
  const float* l_mu;
  uint32_t xoff[NI];
  auto cursor_tile = [&](uint32_t b) __attribute__((always_inline)) {
    lj = next_cblk_job(a, lj, b);
    const JobDesc& jd = a.jobs[lj];
    CSlot& sl = slot_of(a, jd.slot);
    lbe = tile_end(lj, b);
    const uint32_t t0 = (b - jd.cblk_begin) * kEncBlk;
    const uint32_t n = min((lbe - b) * kEncBlk, jd.tc - t0);
    l_venc = (const uint16_t*)(a.state + sl.venc_off);
    l_mu = (const float*)(a.state + sl.mhi_off);
    l_x = (const uint8_t*)jd.src + (size_t)(jd.s1 + t0) * row_bytes;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const uint32_t r = (uint32_t)(wave * 32 + i * RPI + lane / CH);
      xoff[i] = (r < n ? r : 0u) * (uint32_t)row_bytes + (uint32_t)cx * 16u;
    }
  };
  auto cursor_next = [&]() __attribute__((always_inline)) {
    if (lk + 1 < n_sl) {
      ++lk;
    } else if (lbe < b_end) {
      lk = 0;
      cursor_tile(lbe);
    }
  };
  cursor_tile(b_begin);

  // Slice copy: a slice holds 32 * NB rows of kEncKS features, 32 * NB * 8
  // vectors of 16 bytes, so thread t moves vectors t + q * kThreads, q < NB,
  // with no predicate. Every job of a launch has r_enc = 32 * NB; rows >=
  // r_eff are zero in the device state.
  typedef uint32_t vregs_t __attribute__((ext_vector_type(4 * NB)));
#define KVTC_LOAD_SLICE(V)                                                              \
  _Pragma("unroll") for (int q = 0; q < NB; ++q) {                                      \
    const int idx = (int)threadIdx.x + q * kThreads;                                    \
    const uint4 v = *(const uint4*)(l_venc + (size_t)(idx / (kEncKS / 8)) * F +          \
                                    lk * kEncKS + (idx % (kEncKS / 8)) * 8);            \
    V[4 * q] = v.x;                                                                     \
    V[4 * q + 1] = v.y;                                                                 \
    V[4 * q + 2] = v.z;                                                                 \
    V[4 * q + 3] = v.w;                                                                 \
  }
#define KVTC_STORE_SLICE(V, BUF)                                                     \
  _Pragma("unroll") for (int q = 0; q < NB; ++q) {                                   \
    const int idx = (int)threadIdx.x + q * kThreads;                                 \
    *(uint4*)((BUF) + (idx / (kEncKS / 8)) * kEncRowPad + (idx % (kEncKS / 8)) * 8) = \
        make_uint4(V[4 * q], V[4 * q + 1], V[4 * q + 2], V[4 * q + 3]);              \
  }
  // Token rows are read once: non-temporal loads keep them from displacing
  // the basis and the decode's lines in the caches.
#define KVTC_LOAD_X(DST) \
  _Pragma("unroll") for (int i = 0; i < NI; ++i) DST[i] = __builtin_nontemporal_load((const u32x4*)(l_x + xoff[i] + (size_t)lk * kEncKS * esz));
  // Rows of one slice into the wave's token tile as loaded: row
  // i * RPI + lane / CH, features cx * EPC .. + EPC.
  auto stage_x = [&](const u32x4 (&xr)[NI]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NI; ++i) *(u32x4*)(xs + (i * RPI + lane / CH) * XROW + cx * 16) = xr[i];
  };
  // Slice 0 of a tile: its job's centring vector (when it changes), basis and
  // token rows.
  const float* mu_staged = nullptr;
  auto stage_first = [&](const float* mu, const u32x4 (&xr)[NI], const vregs_t& v)
      __attribute__((always_inline)) {
    if (!FOLD && mu != mu_staged) {   // uniform
      for (int i = threadIdx.x; i < F / 4; i += kThreads) ((float4*)mu_l)[i] = ((const float4*)mu)[i];
      __syncthreads();
      mu_staged = mu;
    }
    stage_x(xr);
    KVTC_STORE_SLICE(v, vbase)
    __syncthreads();
  };

  // acc[b][i] holds component 32b + 8(i/4) + 4h + i%4 of token tl. It
  // starts at -(mu32 - mu_hi) V', the part of the mean the centring on
  // mu_hi leaves.
  f32x16 acc[NB];
  auto init_acc = [&](int j) __attribute__((always_inline)) {
    // Scalar loads (constant address space): items 32b + 8q + e of the low
    // half-wave, + 4 for the high one.
    CSlot& sl = slot_of(a, a.jobs[j].slot);
    CU32* cmu = (CU32*)(a.state + sl.cmu_off);
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float lo = __uint_as_float(cmu[32 * b + 8 * q + e]);
          const float hi = __uint_as_float(cmu[32 * b + 8 * q + 4 + e]);
          acc[b][4 * q + e] = -(h ? hi : lo);
        }
  };
  // One slice: run the K steps of slice it (token tile, basis buffer it % 2;
  // K step s takes features 16s + 8h .. +8 of the slice), issue the loads at
  // the load cursor (basis into vl, tokens into xl, both free since the end
  // of slice it - 1; mul is the mean of the tile they belong to), then,
  // unless it is the tile's last slice,
  // stage slice it + 1 (tokens xn, basis vs). The caller alternates the
  // register sets, so no register is copied and every wait is for loads
  // issued one slice earlier.
  auto step = [&](int it, const u32x4 (&xn)[NI], u32x4 (&xl)[NI], vregs_t& vl, vregs_t& vs,
                  const float*& mul) __attribute__((always_inline)) {
    const uint16_t* vsl = vbase + (it & 1) * slice_elems;
    const uint8_t* xrow = xs + (lane & 31) * XROW;
#pragma unroll
    for (int s = 0; s < kEncKS / 16; ++s) {
      // B fragment: features f .. f + 8 of the slice for token lane % 32.
      const int f = 16 * s + 8 * h;
      bf16x8 bx[NT];
      if constexpr (FOLD) {
        bx[0] = __builtin_bit_cast(bf16x8, *(const u32x4*)(xrow + 2 * f));
      } else {
        const float4 m0 = *(const float4*)(mu_l + it * kEncKS + f);
        const float4 m1 = *(const float4*)(mu_l + it * kEncKS + f + 4);
        const float mv[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
        float d[8];
        if (F32IN) {
          const u32x4 x0 = *(const u32x4*)(xrow + 4 * f);
          const u32x4 x1 = *(const u32x4*)(xrow + 4 * f + 16);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            d[e] = __uint_as_float(x0[e]) - mv[e];
            d[e + 4] = __uint_as_float(x1[e]) - mv[e + 4];
          }
        } else {   // two bf16 per dword, low half first
          const u32x4 x0 = *(const u32x4*)(xrow + 2 * f);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            d[2 * e] = __uint_as_float(x0[e] << 16) - mv[2 * e];
            d[2 * e + 1] = __uint_as_float(x0[e] & 0xFFFF0000u) - mv[2 * e + 1];
          }
        }
#pragma unroll
        for (int p = 0; p < NT; ++p) {
          uint32_t t[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            t[e] = pack_bf16x2(d[2 * e], d[2 * e + 1]);
            if (p + 1 < NT) {   // the remainder is exact in fp32
              d[2 * e] -= bf16_to_f32(t[e] & 0xFFFFu);
              d[2 * e + 1] -= bf16_to_f32(t[e] >> 16);
            }
          }
          bx[p] = __builtin_bit_cast(bf16x8, (u32x4){t[0], t[1], t[2], t[3]});
        }
      }
      bf16x8 av[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b)
        av[b] = __builtin_bit_cast(bf16x8, *(const uint4*)(vsl + (b * 32 + (lane & 31)) * kEncRowPad + f));
      // term-major: consecutive MFMAs go to different accumulators
#pragma unroll
      for (int p = 0; p < NT; ++p)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[b], bx[p], acc[b], 0, 0, 0);
    }
    // The loads go after the MFMA issue: when the memory pipeline is backed
    // up, issuing them stalls the wave, and the MFMAs then run meanwhile.
    __builtin_amdgcn_sched_barrier(0);
    KVTC_LOAD_SLICE(vl)
    KVTC_LOAD_X(xl)
    mul = l_mu;
    cursor_next();
    // The token tile is private to the wave: its reads above come before the
    // writes below in the wave's LDS order. After a tile's last slice this
    // stages the next tile's slice 0, which the records then overwrite; it
    // is staged again from the same registers after them.
    wave_lds_sync();
    stage_x(xn);
    KVTC_STORE_SLICE(vs, vbase + ((it + 1) & 1) * slice_elems)
    __syncthreads();
  };

  u32x4 x0[NI], x1[NI];
  vregs_t v0, v1;
  const float *mu0 = l_mu, *mu1;   // the mean of the tile in x0 / x1
  KVTC_LOAD_SLICE(v0)
  KVTC_LOAD_X(x0)
  cursor_next();
  mu1 = l_mu;
  KVTC_LOAD_SLICE(v1)
  KVTC_LOAD_X(x1)
  cursor_next();
  init_acc(j_begin);
  stage_first(mu0, x0, v0);
  int cj = j_begin;   // the computed tile's job
  for (uint32_t b = b_begin, te; b < b_end; b = te) {
    cj = next_cblk_job(a, cj, b);
    te = tile_end(cj, b);
    const JobDesc& jd = a.jobs[cj];
    CSlot& sl = slot_of(a, jd.slot);
    const uint32_t t0 = (b - jd.cblk_begin) * kEncBlk;
    const uint32_t n = min((te - b) * kEncBlk, jd.tc - t0);
    // The loop runs whole pairs of steps and an odd last slice follows it,
    // so the loop is only re-entered after a pair; with the parity fixed at
    // compile time every path into the loop has the same loads in flight and
    // the waits the compiler derives at its head cover just those.
    int it = 0;
    for (; it + 1 < n_sl; it += 2) {
      step(it, x1, x0, v0, v1, mu0);
      step(it + 1, x0, x1, v1, v0, mu1);
    }
    if (ODD) step(it, x1, x0, v0, v1, mu0);
    __syncthreads();  // every wave is done with the slices in LDS
    const int rb = sl.record_bytes;
    const int rbp = padded_stride(rb);
    {
      // Zero the wave's 32 record rows (16-byte aligned: rbp % 4 == 0).
      u32x4* z = (u32x4*)(smem + (size_t)wave * 32 * rbp);
      const int nz = 32 * rbp / 16;
      for (int i = lane; i < nz; i += 64) z[i] = (u32x4){0u, 0u, 0u, 0u};
      wave_lds_sync();
    }
    quantize_tile<NB, G>(acc, sl, a.state, smem + (size_t)tl * rbp, h, (uint32_t)tl < n);
    if (te < b_end) init_acc(next_cblk_job(a, cj, te));
    __syncthreads();
    records_to_global((uint8_t*)jd.dst + record_base(jd, F, esz) + (size_t)t0 * rb, smem, n, rb, rbp);
    if (te < b_end) {
      __syncthreads();  // the records are out of LDS
      if (ODD) {
        // Odd slice count: the next tile's slice 0 is in (x1, v1), slice 1
        // in (x0, v0); swap so the tile starts like the first one.
        stage_first(mu1, x1, v1);
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const u32x4 t = x0[i];
          x0[i] = x1[i];
          x1[i] = t;
        }
        const vregs_t t = v0;
        v0 = v1;
        v1 = t;
        mu1 = mu0;
      } else {
        stage_first(mu0, x0, v0);
      }
    }
  }
#undef KVTC_LOAD_SLICE
#undef KVTC_STORE_SLICE
#undef KVTC_LOAD_X
}

// Test hook: stream from given codes and (shift, scale) pairs, through the
// encoder's record packing (the same lane layout, or_code_run, put_scales and
// records_to_global) and header/passthrough writers.
template <int G>
__global__ __launch_bounds__(kThreads) void pack_kernel(const LaunchArgs a, const uint8_t* codes,
                                                        const float2* ss) {
  extern __shared__ __align__(16) uint8_t smem[];
  const uint32_t tile = logical_tile();
  if (tile >= a.total_tiles) return;
  const JobDesc& jd = a.jobs[0];
  CSlot& sl = slot_of(a, jd.slot);
  const uint32_t lt = tile - jd.tile_begin;
  const int esz = a.dtype == KVTC_F32 ? 4 : 2;
  const size_t row_bytes = (size_t)a.F * esz;
  if (lt == 0 && threadIdx.x == 0) {
    write_header(a, jd, sl);
    set_status(a, jd.status_idx, KVTC_OK);
  }
  if (lt >= jd.n_ctiles) {
    encode_passthrough(jd, lt - jd.n_ctiles, row_bytes);
    return;
  }
  if (sl.r_eff == 0) return;
  const uint32_t t0 = lt * kEncTile;
  const uint32_t n = min((uint32_t)kEncTile, jd.tc - t0);
  const int rb = sl.record_bytes;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5;
  const int tl = wave * 32 + (lane & 31);
  const int rbp = padded_stride(rb);
  {
    // Zero the workgroup's record rows (16-byte aligned: rbp % 4 == 0).
    u32x4* z = (u32x4*)smem;
    for (int i = threadIdx.x; i < kEncTile * rbp / 16; i += kThreads) z[i] = (u32x4){0u, 0u, 0u, 0u};
  }
  __syncthreads();
  if ((uint32_t)tl < n) {
    // The lane layout of the encode (quantize_tile): lane half h holds, of
    // each group, the runs of four components 8m + 4h .. + 3.
    const uint32_t t = t0 + tl;
    uint32_t* rw = (uint32_t*)(smem + (size_t)tl * rbp);
    for (int ag = 0; ag < sl.n_act; ++ag) {
      const int w = slot_width(sl, ag);
      for (int m = 0; m < G / 8; ++m) {
        const int o = 8 * m + 4 * h;
        uint32_t run = 0;
        for (int e = 0; e < 4; ++e) run |= (uint32_t)codes[(size_t)t * sl.r_eff + ag * G + o + e] << (e * w);
        or_code_run(rw, code_bit(sl, ag, o, w), run, w);
      }
      const float2 p = ss[(size_t)t * sl.n_act + ag];
      if (h == 0) put_scales(rw, ag, p.x, p.y);
    }
  }
  __syncthreads();
  records_to_global((uint8_t*)jd.dst + record_base(jd, a.F, esz) + (size_t)t0 * rb, smem, n, rb, rbp);
}


// ------------------------------------------------------------- launchers ---

// Encode workgroups per CU: the per-CU load throughput saturates at two
// (measured on llama31_8b, 32 tensors: 174 us per launch at one per CU,
// 143 at two, 150 at three).
constexpr int kEncMaxPerCU = 2;

template <int G, bool F32IN, bool ODD, bool FOLD>
static int launch_encode_g(const LaunchArgs& a, int nb, size_t lds, hipStream_t s) {
  // Persistent: the resident workgroups (at most kEncMaxPerCU per CU), or
  // fewer when there are fewer compressed blocks (any grid covers the
  // headers and passthrough units).
#define KVTC_ENC(NBV)                                                                      \
  case NBV: {                                                                              \
    allow_lds(encode_kernel<NBV, G, F32IN, ODD, FOLD>, lds);                                     \
    const dim3 g(std::min({grid_for(std::max(1u, (a.total_cblks + kEncWaves - 1) / kEncWaves)).x, \
                           resident_grid(encode_kernel<NBV, G, F32IN, ODD, FOLD>, kThreads, lds,  \
                                         kEncMaxPerCU),                                    \
                           persistent_grid_cap()}));                                           \
    hipLaunchKernelGGL((encode_kernel<NBV, G, F32IN, ODD, FOLD>), g, dim3(kThreads), lds, s, a); \
    break;                                                                                 \
  }
  switch (nb) {
    KVTC_ENC(1) KVTC_ENC(2) KVTC_ENC(3) KVTC_ENC(4) KVTC_ENC(5) KVTC_ENC(6) KVTC_ENC(7) KVTC_ENC(8)
    default:
      return (int)hipErrorInvalidValue;
  }
#undef KVTC_ENC
  return (int)hipGetLastError();
}

int launch_encode(const LaunchArgs& a, int nb, int G, size_t lds, hipStream_t s) {
  const bool f32 = a.dtype == KVTC_F32;
  const bool odd = (a.F / kEncKS) & 1;
  if (f32 && a.fold) return (int)hipErrorInvalidValue;
#define KVTC_ENC_G(GV)                                                                   \
  if (G == GV)                                                                           \
    return f32 ? (odd ? launch_encode_g<GV, true, true, false>(a, nb, lds, s)            \
                      : launch_encode_g<GV, true, false, false>(a, nb, lds, s))          \
               : a.fold ? (odd ? launch_encode_g<GV, false, true, true>(a, nb, lds, s)   \
                               : launch_encode_g<GV, false, false, true>(a, nb, lds, s)) \
                        : (odd ? launch_encode_g<GV, false, true, false>(a, nb, lds, s)  \
                               : launch_encode_g<GV, false, false, false>(a, nb, lds, s));
  KVTC_ENC_G(16)
  KVTC_ENC_G(32)
#undef KVTC_ENC_G
  return (int)hipErrorInvalidValue;
}

// Decode launches take the exact K-step count ks = r_dec / 16 of every job
// in the batch (the host groups jobs by it).
int launch_pack(const LaunchArgs& a, int G, size_t lds, const void* codes, const void* ss,
                hipStream_t s) {
  const dim3 g = grid_for(a.total_tiles);
  if (G == 16)
    hipLaunchKernelGGL((pack_kernel<16>), g, dim3(kThreads), lds, s, a, (const uint8_t*)codes,
                       (const float2*)ss);
  else if (G == 32)
    hipLaunchKernelGGL((pack_kernel<32>), g, dim3(kThreads), lds, s, a, (const uint8_t*)codes,
                       (const float2*)ss);
  else
    return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}

}  // namespace kvtc
