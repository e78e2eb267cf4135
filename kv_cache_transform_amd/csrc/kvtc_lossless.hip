// Lossless stage of libkvtc for gfx950: a KVTC stream <-> a KVTZ container.
//
// The KVTC page (section 2B) finishes compression with DEFLATE on the GPU.
// This stage is our own replacement that knows the stream's layout: the
// stream is split into fields (passthrough byte planes, the byte planes of
// the fp32 shifts and scales, one field of codes per active group), each
// field gets a static model (its histogram normalised to kLzM), and each
// field is coded by rANS (range asymmetric numeral systems, J. Duda) in
// independent chunks of kLzChunk symbols. A chunk has 64 interleaved states
// and is coded by one wavefront, one state per lane: each step codes 64
// consecutive symbols, and the words the step emits or takes are placed by a
// ballot and a prefix count. The container layout is written out in kvtc.h
// at kvtc_lossless_encode.
//
// Encode: split (stream -> field symbols), histogram, model (normalise,
// write the tables), code (one wavefront per chunk, words into scratch), layout
// (per job: chunk directory by a prefix sum, container header), copy
// (payloads in decoder order). Decode: check (container header, tables,
// directory), model (slot tables), decode (one wavefront per chunk),
// merge (field symbols -> stream). Every kernel is memory- or latency-bound;
// no matrix unit is involved.
#include "kvtc_device.h"

namespace kvtc {
namespace {

constexpr int kLzThreads = 256;

template <uint32_t LzJob::*M>
__device__ __forceinline__ int lz_job_at(const LzArgs& a, uint32_t x) {
  int lo = 0, hi = a.n_jobs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.jobs[mid].*M <= x) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ const DevSlot* lz_slot(const LzArgs& a, const LzJob& j) {
  return (const DevSlot*)a.state + j.slot;
}

__device__ __forceinline__ LzShape lz_shape(const LzArgs& a, const LzJob& j) {
  const DevSlot* sl = lz_slot(a, j);
  LzShape s;
  s.esz = a.esz;
  s.n_act = sl->n_act;
  s.G = sl->G;
  s.n_pt = (j.s1 + j.w1) * (uint32_t)a.F;
  s.tc = j.tc;
  s.width = sl->width;
  return s;
}

__device__ __forceinline__ void lz_set(const LzArgs& a, const LzJob& j, int st) {
  atomicMax(&a.status[j.status_idx], ((unsigned long long)a.epoch << 32) | (unsigned long long)status_rank(st));
}

// True if an earlier kernel of this call found the job bad.
__device__ __forceinline__ bool lz_failed(const LzArgs& a, const LzJob& j) {
  const unsigned long long w = __atomic_load_n(&a.status[j.status_idx], __ATOMIC_RELAXED);
  return (uint32_t)(w >> 32) == a.epoch && (w & 0xFFull) != 0;
}

// Where field f's symbols start, for the fields whose position is a
// closed form: the planes (f < esz + 8) and the first code field.
__device__ __forceinline__ uint32_t lz_plane_off(const LzShape& s, int f) {
  const uint32_t rp = lz_sym_region(s.n_pt), rs = lz_sym_region(s.tc * (uint32_t)s.n_act);
  return f < s.esz ? f * rp : s.esz * rp + (f - s.esz) * rs;
}
__device__ __forceinline__ uint32_t lz_code_off(const LzShape& s, int a) {
  return lz_plane_off(s, s.esz + 8) + a * lz_sym_region(s.tc * (uint32_t)s.G);
}

// Wave-wide (64 lanes) reductions and an inclusive scan.
__device__ __forceinline__ uint64_t wave_sum(uint64_t v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
  for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
  return v;
}
__device__ __forceinline__ uint32_t wave_min(uint32_t v) {
  for (int o = 32; o > 0; o >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, o, 64));
  return v;
}
__device__ __forceinline__ uint32_t wave_scan(uint32_t v, int lane) {
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t u = (uint32_t)__shfl_up((int)v, o, 64);
    if (lane >= o) v += u;
  }
  return v;
}

// ------------------------------------------------------------- encode ----

// One unit: a block of kLzPassBlk passthrough elements, or of kLzRecBlk
// records, written out as field symbols. Unit 0 of a job also marks the job
// OK for this call and clears its histograms.
__global__ void __launch_bounds__(kLzThreads) lz_split_kernel(const LzArgs a) {
  extern __shared__ uint8_t lds[];
  const int ji = lz_job_at<&LzJob::unit0>(a, blockIdx.x);
  const LzJob& j = a.jobs[ji];
  const LzShape s = lz_shape(a, j);
  const uint32_t u = blockIdx.x - j.unit0;
  const int tid = threadIdx.x;
  if (u == 0) {
    if (tid == 0) lz_set(a, j, KVTC_OK);
    const LzLayout L = lz_layout(s, true);
    uint32_t* h = (uint32_t*)(j.ws + L.hist);
    for (int i = tid; i < lz_nf(s) * 256; i += kLzThreads) h[i] = 0;
  }
  const uint32_t n_pb = (s.n_pt + kLzPassBlk - 1) / kLzPassBlk;
  uint8_t* sym = j.ws;
  if (u < n_pb) {
    // 16 consecutive elements a thread: 16-byte loads of the stream (its
    // passthrough rows start at byte 64) and a 16-byte store per plane
    const uint32_t e0 = u * kLzPassBlk + 16 * tid;
    if (e0 >= s.n_pt) return;
    const uint8_t* src = j.src + kHeaderBytes + (size_t)e0 * s.esz;
    const uint32_t rp = lz_sym_region(s.n_pt);
    if (e0 + 16 <= s.n_pt) {
      u32x4 pl[4] = {u32x4(0u), u32x4(0u), u32x4(0u), u32x4(0u)};
      for (int v = 0; v < s.esz; ++v) {                 // 4 (bf16) or 8 (f32) elements per load
        const u32x4 w = ((const u32x4*)src)[v];
        for (int q = 0; q < 4; ++q) {
          if (s.esz == 2) {
            const int e = 8 * v + 2 * q;                // elements e, e + 1 of the 16
            pl[0][e >> 2] |= ((w[q] & 0xFFu) | ((w[q] >> 8) & 0xFF00u)) << (8 * (e & 3));
            pl[1][e >> 2] |= (((w[q] >> 8) & 0xFFu) | ((w[q] >> 16) & 0xFF00u)) << (8 * (e & 3));
          } else {
            const int e = 4 * v + q;
            for (int b = 0; b < 4; ++b) pl[b][e >> 2] |= ((w[q] >> (8 * b)) & 0xFFu) << (8 * (e & 3));
          }
        }
      }
      for (int b = 0; b < s.esz; ++b) *(u32x4*)(sym + b * rp + e0) = pl[b];
    } else {
      for (uint32_t e = e0; e < s.n_pt; ++e) {
        const uint8_t* p = j.src + kHeaderBytes + (size_t)e * s.esz;
        for (int b = 0; b < s.esz; ++b) sym[b * rp + e] = p[b];
      }
    }
    return;
  }
  const uint32_t r0 = (u - n_pb) * kLzRecBlk;
  if (r0 >= s.tc) return;
  const DevSlot* sl = lz_slot(a, j);
  const int rb = sl->record_bytes, na = s.n_act, G = s.G;
  const int nr = (int)min((uint32_t)kLzRecBlk, s.tc - r0);
  // the block's records into LDS (16-byte aligned: the records start at
  // 64 + n_pt * esz, a multiple of 16, and a block at 64 * rb bytes)
  const uint8_t* base = j.src + kHeaderBytes + (size_t)s.n_pt * s.esz + (size_t)r0 * rb;
  const int nbytes = nr * rb;
  for (int i = tid * 4; i + 4 <= nbytes; i += kLzThreads * 4) *(uint32_t*)(lds + i) = *(const uint32_t*)(base + i);
  for (int i = (nbytes & ~3) + tid; i < nbytes; i += kLzThreads) lds[i] = base[i];
  __syncthreads();
  // every field's run of this block starts at a multiple of 4 (r0 is a
  // multiple of 64); a thread writes 4 consecutive symbols. A run only ends
  // inside a word in the field's last block, where the zeros past its end
  // land in the region's padding.
  for (int k = 0; k < 8; ++k) {
    uint8_t* out = sym + lz_plane_off(s, s.esz + k) + (size_t)r0 * na;
    for (int i = 4 * tid; i < nr * na; i += 4 * kLzThreads) {
      uint32_t v = 0;
      int t = i / na, g = i - t * na;
      for (int q = 0; q < 4 && i + q < nr * na; ++q) {
        v |= (uint32_t)lds[t * rb + g * 8 + k] << (8 * q);
        if (++g == na) {
          g = 0;
          ++t;
        }
      }
      *(uint32_t*)(out + i) = v;
    }
  }
  // With a width per component, code j of active group g sits at the record
  // bit and width of the slot's table entry g * G + j ((bit << 8) | width).
  const uint32_t* pcw = sl->pc ? (const uint32_t*)(a.state + sl->pcw_off) : nullptr;
  for (int g = 0; g < na; ++g) {
    const int b = s.width[g], co = sl->chunk_off[g];
    const uint32_t mask = (1u << b) - 1u;
    uint8_t* out = sym + lz_code_off(s, g) + (size_t)r0 * G;
    for (int i = 4 * tid; i < nr * G; i += 4 * kLzThreads) {
      const int t = i / G, c = i - t * G;      // G is a multiple of 8: one record
      uint32_t v = 0;
      for (int q = 0; q < 4; ++q) {
        int bit = 8 * co + (c + q) * b;
        uint32_t m = mask;
        if (pcw) {
          const uint32_t e = pcw[g * G + c + q];
          bit = (int)(e >> 8);
          m = (1u << (e & 0xFFu)) - 1u;
        }
        const int p = t * rb + (bit >> 3);
        const uint32_t w = ((uint32_t)lds[p] | ((uint32_t)lds[p + 1] << 8)) >> (bit & 7);
        v |= (w & m) << (8 * q);
      }
      *(uint32_t*)(out + i) = v;
    }
  }
}

// One unit: kLzSeg symbols of one field into the field's histogram (a
// sub-histogram per wave in LDS, runs of equal symbols added at once).
__global__ void __launch_bounds__(kLzThreads) lz_hist_kernel(const LzArgs a) {
  __shared__ uint32_t h[kLzThreads / 64][256];
  const int ji = lz_job_at<&LzJob::seg0>(a, blockIdx.x);
  const LzJob& j = a.jobs[ji];
  const LzShape s = lz_shape(a, j);
  const uint32_t u = blockIdx.x - j.seg0;
  uint32_t seg0 = 0, sym_off = 0;
  int f = 0;
  for (; f < lz_nf(s); ++f) {
    const uint32_t nf = lz_n(s, f), ns = (nf + kLzSeg - 1) / kLzSeg;
    if (u < seg0 + ns) break;
    seg0 += ns;
    sym_off += lz_sym_region(nf);
  }
  const int tid = threadIdx.x, w = tid >> 6;
  for (int i = tid; i < 256 * (kLzThreads / 64); i += kLzThreads) (&h[0][0])[i] = 0;
  __syncthreads();
  const uint32_t n = lz_n(s, f);
  const uint32_t b0 = (u - seg0) * kLzSeg, b1 = min(n, b0 + kLzSeg);
  const uint8_t* sym = j.ws + sym_off;
  for (uint32_t i = b0 + tid * 16; i < b1; i += kLzThreads * 16) {
    const u32x4 v = *(const u32x4*)(sym + i);
    const int m = (int)min(16u, b1 - i);
    uint32_t cur = v[0] & 0xFFu, run = 0;
    for (int k = 0; k < m; ++k) {
      const uint32_t c = (v[k >> 2] >> (8 * (k & 3))) & 0xFFu;
      if (c != cur) {
        atomicAdd(&h[w][cur], run);
        cur = c;
        run = 0;
      }
      ++run;
    }
    atomicAdd(&h[w][cur], run);
  }
  __syncthreads();
  uint32_t t = 0;
  for (int k = 0; k < kLzThreads / 64; ++k) t += h[k][tid];
  if (t) {
    const LzLayout L = lz_layout(s, true);
    atomicAdd((uint32_t*)(j.ws + L.hist) + f * 256 + tid, t);
  }
}

// One wave per field: normalise the histogram (every present symbol gets
// 1 + floor(h * (M - n_present) / N), the remainder goes to the most
// frequent symbol, lowest index on ties), write the container's table entry
// and the coder's model (f | c << 16 and a 32-bit reciprocal of f).
__global__ void __launch_bounds__(64) lz_model_kernel(const LzArgs a) {
  const int ji = lz_job_at<&LzJob::field0>(a, blockIdx.x);
  const LzJob& j = a.jobs[ji];
  const LzShape s = lz_shape(a, j);
  const int f = blockIdx.x - j.field0, lane = threadIdx.x;
  const uint32_t n = lz_n(s, f);
  const int A = lz_alpha(s, f);
  const LzField fd = lz_field(s, f);
  const LzLayout L = lz_layout(s, true);
  uint8_t* tab = j.dst + fd.tab_off;
  if (lane == 0) {
    *(uint32_t*)tab = n;
    *(uint32_t*)(tab + 4) = (uint32_t)A;
  }
  const uint32_t* hist = (const uint32_t*)(j.ws + L.hist) + f * 256;
  uint32_t* fc = (uint32_t*)(j.ws + L.fc) + f * 256;
  uint32_t* rcp = (uint32_t*)(j.ws + L.aux) + f * 256;
  uint32_t hv[4], fv[4];
  uint64_t N = 0;
  uint32_t np = 0, hmax = 0;
  for (int q = 0; q < 4; ++q) {
    const int sy = lane + 64 * q;
    hv[q] = sy < A ? hist[sy] : 0;
    N += hv[q];
    np += hv[q] ? 1 : 0;
    hmax = max(hmax, hv[q]);
  }
  N = wave_sum(N);
  np = (uint32_t)wave_sum(np);
  hmax = wave_max(hmax);
  uint32_t first = 256;
  for (int q = 3; q >= 0; --q)
    if (hv[q] == hmax && hmax) first = lane + 64 * q;
  first = wave_min(first);
  uint32_t sum = 0;
  for (int q = 0; q < 4; ++q) {
    fv[q] = hv[q] ? 1u + (uint32_t)(((uint64_t)hv[q] * (kLzM - np)) / (N ? N : 1)) : 0u;
    sum += fv[q];
  }
  sum = (uint32_t)wave_sum(sum);
  if (N)
    for (int q = 0; q < 4; ++q)
      if ((uint32_t)(lane + 64 * q) == first) fv[q] += kLzM - sum;
  uint32_t run = 0;
  for (int q = 0; q < 4; ++q) {
    const int sy = lane + 64 * q;
    const uint32_t inc = wave_scan(fv[q], lane);
    const uint32_t c = run + inc - fv[q];
    run += (uint32_t)__shfl((int)inc, 63, 64);
    if (sy < A) {
      ((uint16_t*)(tab + 8))[sy] = (uint16_t)fv[q];
      fc[sy] = fv[q] | (c << 16);
      // floor(2^32 / f) (2^32 - 1 for f = 1): x * rcp >> 32 is floor(x / f)
      // or one less, for every 32-bit x
      rcp[sy] = fv[q] > 1 ? (uint32_t)(0x100000000ull / fv[q]) : 0xFFFFFFFFu;
    }
  }
}

__device__ __forceinline__ uint64_t lanes_below(int l) { return (1ull << l) - 1ull; }

// One wavefront per chunk: the steps from the last to the first, lane l
// coding symbol 64 t + l with its own state. The field's model (f | c << 16
// and the reciprocal of f, one 8-byte entry per symbol) is staged in LDS,
// and the chunk's symbols half a chunk at a time (the upper half first), so
// a workgroup holds 10 KiB of LDS and every chunk of a launch can be
// resident at once. Within a half the next step's symbol and entry are
// read one step ahead, so the loop's chain is the state arithmetic alone
// and it issues no global load (only the stores of emitted words, which
// nothing waits for). A step's emitted words go to the chunk's scratch in
// reverse decoder order (the copy kernel reverses them): the k words of a
// step take the next k positions, the lane of rank r among the emitting
// lanes position k - 1 - r.
constexpr uint32_t kLzHalf = kLzChunk / 2;   // symbols staged at a time
__global__ void __launch_bounds__(kLzLanes) lz_code_kernel(const LzArgs a) {
  __shared__ __align__(16) uint8_t syms[kLzHalf];
  __shared__ uint64_t mdl[256];
  const uint32_t g = blockIdx.x;
  const int l = threadIdx.x;
  const int ji = lz_job_at<&LzJob::chunk0>(a, g);
  const LzJob& j = a.jobs[ji];
  const LzShape s = lz_shape(a, j);
  const uint32_t kj = g - j.chunk0;
  uint32_t k = kj, sym_off = 0;
  int f = 0;
  for (; f < lz_nf(s); ++f) {
    const uint32_t nc = lz_chunks(lz_n(s, f));
    if (k < nc) break;
    k -= nc;
    sym_off += lz_sym_region(lz_n(s, f));
  }
  const LzLayout L = lz_layout(s, true);
  const uint32_t len = min((uint32_t)kLzChunk, lz_n(s, f) - k * kLzChunk);
  // (the field's symbol region is padded: whole 16-byte reads stay inside)
  const u32x4* src = (const u32x4*)(j.ws + sym_off + (size_t)k * kLzChunk);
  const uint32_t* fc = (const uint32_t*)(j.ws + L.fc) + f * 256;
  const uint32_t* rcp = (const uint32_t*)(j.ws + L.aux) + f * 256;
  for (int i = l; i < 256; i += kLzLanes) mdl[i] = fc[i] | ((uint64_t)rcp[i] << 32);
  uint16_t* rev = (uint16_t*)(j.ws + L.scratch) + (size_t)kj * kLzChunk;
  uint32_t x = kLzL, cnt = 0;
  constexpr int kHalfSteps = (int)(kLzHalf / kLzLanes);
  const int steps = (int)((len + kLzLanes - 1) / kLzLanes);
  for (int hf = (steps - 1) / kHalfSteps; hf >= 0; --hf) {
    const int t0 = hf * kHalfSteps;
    const uint32_t n16 = (min(len - (uint32_t)t0 * kLzLanes, kLzHalf) + 15) / 16;
    __syncthreads();   // the previous half's reads are done
    for (uint32_t i = l; i < n16; i += kLzLanes) ((u32x4*)syms)[i] = src[(uint32_t)t0 * kLzLanes / 16 + i];
    __syncthreads();
    int t = min(steps, t0 + kHalfSteps) - 1;
    // only the chunk's last step can be partial
    bool act = (uint32_t)t * kLzLanes + l < len;
    uint64_t m = mdl[act ? syms[(uint32_t)(t - t0) * kLzLanes + l] : 0u];
    for (; t >= t0; --t) {
      const uint64_t mn = t > t0 ? mdl[syms[(uint32_t)(t - 1 - t0) * kLzLanes + l]] : 0ull;
      const uint32_t fs = (uint32_t)m & 0xFFFFu, cs = ((uint32_t)m >> 16) & 0xFFFFu, rf = (uint32_t)(m >> 32);
      const bool emit = act && (uint64_t)x >= ((uint64_t)fs << 20);
      const uint64_t mask = __ballot(emit);
      const uint32_t ke = (uint32_t)__popcll(mask);
      if (emit) rev[cnt + ke - 1 - (uint32_t)__popcll(mask & lanes_below(l))] = (uint16_t)x;
      cnt += ke;
      const uint32_t xe = emit ? x >> 16 : x;
      uint32_t q = __umulhi(xe, rf);
      uint32_t rm = xe - q * fs;
      const bool up = rm >= fs;
      q += up ? 1u : 0u;
      rm -= up ? fs : 0u;
      x = act ? (q << kLzMBits) + rm + cs : x;
      m = mn;
      act = true;
    }
  }
  ((uint32_t*)(j.ws + L.state))[(size_t)kj * kLzLanes + l] = x;
  if (l == 0) ((uint32_t*)(j.ws + L.cnt))[kj] = cnt;
}

// One workgroup per job: payload sizes -> chunk directory (prefix sum) and
// payload offsets; the container header, the stream header, the padding.
__global__ void __launch_bounds__(kLzThreads) lz_layout_kernel(const LzArgs a) {
  __shared__ uint32_t part[kLzThreads / 64];
  const LzJob& j = a.jobs[blockIdx.x];
  const LzShape s = lz_shape(a, j);
  const LzLayout L = lz_layout(s, true);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const uint32_t* cnt = (const uint32_t*)(j.ws + L.cnt);
  uint32_t* dsto = (uint32_t*)(j.ws + L.dsto);
  uint32_t* dir = (uint32_t*)(j.dst + L.dir_off);
  uint32_t run = 0;
  for (uint32_t k0 = 0; k0 < L.n_chunks; k0 += kLzThreads) {
    const uint32_t k = k0 + tid;
    const uint32_t bytes = k < L.n_chunks ? 4 * kLzLanes + 2 * cnt[k] : 0;
    const uint32_t inc = wave_scan(bytes, lane);
    if (lane == 63) part[w] = inc;
    __syncthreads();
    uint32_t before = run;
    for (int q = 0; q < w; ++q) before += part[q];
    uint32_t tile = 0;
    for (int q = 0; q < kLzThreads / 64; ++q) tile += part[q];
    if (k < L.n_chunks) {
      dir[k] = before + inc;
      dsto[k] = before + inc - bytes;
    }
    run += tile;
    __syncthreads();
  }
  const uint32_t end = L.pay_off + run;
  const uint64_t total = (end + 15u) & ~15u;
  if (tid < 16) {
    uint32_t v = 0;
    switch (tid) {
      case 0: v = 0x5A54564Bu; break;                     // "KVTZ"
      case 1: v = 1u | ((uint32_t)lz_nf(s) << 16); break;
      case 2: v = (uint32_t)kLzChunk; break;
      case 3: v = L.n_chunks; break;
      case 4: v = (uint32_t)j.stream_bytes; break;
      case 5: v = (uint32_t)(j.stream_bytes >> 32); break;
      case 6: v = (uint32_t)total; break;
      case 7: v = (uint32_t)(total >> 32); break;
      case 8: v = L.pay_off; break;
      default: v = 0;
    }
    ((uint32_t*)j.dst)[tid] = v;
  } else if (tid < 32) {
    ((uint32_t*)(j.dst + kLzHead))[tid - 16] = ((const uint32_t*)j.src)[tid - 16];
  }
  for (uint32_t i = L.dir_off + 4 * L.n_chunks + tid; i < L.pay_off; i += kLzThreads) j.dst[i] = 0;
  for (uint32_t i = end + tid; i < total; i += kLzThreads) j.dst[i] = 0;
  if (tid == 0) a.sizes[j.status_idx] = total;
}

// One workgroup per chunk: its payload in decoder order (the 64 final
// states, then the words, reversed from the scratch).
__global__ void __launch_bounds__(kLzThreads) lz_copy_kernel(const LzArgs a) {
  const uint32_t g = blockIdx.x;
  const int ji = lz_job_at<&LzJob::chunk0>(a, g);
  const LzJob& j = a.jobs[ji];
  const LzShape s = lz_shape(a, j);
  const LzLayout L = lz_layout(s, true);
  const uint32_t k = g - j.chunk0;
  const uint32_t cnt = ((const uint32_t*)(j.ws + L.cnt))[k];
  const uint32_t off = ((const uint32_t*)(j.ws + L.dsto))[k];
  const uint32_t* st = (const uint32_t*)(j.ws + L.state) + (size_t)k * kLzLanes;
  const uint16_t* sc = (const uint16_t*)(j.ws + L.scratch) + (size_t)k * kLzChunk;
  uint16_t* out = (uint16_t*)(j.dst + L.pay_off + off);
  constexpr uint32_t nst = 2 * kLzLanes;
  for (uint32_t i = threadIdx.x; i < cnt + nst; i += kLzThreads)
    out[i] = i < nst ? (uint16_t)(st[i >> 1] >> (16 * (i & 1))) : sc[cnt - 1 - (i - nst)];
}

// ------------------------------------------------------------- decode ----

// One workgroup per job: the container's header, field table entries and
// chunk directory must be those of the job's shape and self-consistent.
__global__ void __launch_bounds__(kLzThreads) lz_check_kernel(const LzArgs a) {
  __shared__ int bad;
  const LzJob& j = a.jobs[blockIdx.x];
  const LzShape s = lz_shape(a, j);
  const LzLayout L = lz_layout(s, false);
  const int tid = threadIdx.x;
  if (tid == 0) {
    lz_set(a, j, KVTC_OK);
    bad = KVTC_OK;
  }
  __syncthreads();
  const uint32_t* h = (const uint32_t*)j.src;
  const uint64_t total = (uint64_t)h[6] | ((uint64_t)h[7] << 32);
  if (tid == 0) {
    int st = KVTC_OK;
    if (h[0] != 0x5A54564Bu || (h[1] & 0xFFFFu) != 1u || h[2] != (uint32_t)kLzChunk)
      st = KVTC_E_CORRUPT;
    else if ((h[1] >> 16) != (uint32_t)lz_nf(s) || h[3] != L.n_chunks ||
             ((uint64_t)h[4] | ((uint64_t)h[5] << 32)) != j.stream_bytes || h[8] != L.pay_off)
      st = KVTC_E_MISMATCH;
    else if (total % 16 || total > j.src_cap || total < L.pay_off)
      st = KVTC_E_CORRUPT;
    if (st != KVTC_OK) bad = st;
  }
  __syncthreads();
  if (bad != KVTC_OK) {
    if (tid == 0) lz_set(a, j, bad);
    return;
  }
  if (tid < lz_nf(s)) {
    const LzField fd = lz_field(s, tid);
    const uint32_t* e = (const uint32_t*)(j.src + fd.tab_off);
    if (e[0] != lz_n(s, tid) || e[1] != (uint32_t)lz_alpha(s, tid)) atomicMax(&bad, (int)-KVTC_E_MISMATCH);
  }
  const uint32_t* dir = (const uint32_t*)(j.src + L.dir_off);
  for (uint32_t k = tid; k < L.n_chunks; k += kLzThreads) {
    const uint32_t e = dir[k], p = k ? dir[k - 1] : 0;
    if ((e & 1u) || e < p + 4 * kLzLanes || (uint64_t)L.pay_off + e > total) atomicMax(&bad, (int)-KVTC_E_CORRUPT);
  }
  __syncthreads();
  if (tid == 0) {
    const uint32_t last = L.n_chunks ? dir[L.n_chunks - 1] : 0;
    if (((L.pay_off + (uint64_t)last + 15) & ~15ull) != total) atomicMax(&bad, (int)-KVTC_E_CORRUPT);
  }
  __syncthreads();
  if (tid == 0 && bad != KVTC_OK) lz_set(a, j, -bad);
}

// One workgroup per field: the model from the container's table (it must
// sum to M) as the decoder's two tables: per slot its symbol (one byte, kLzM
// bytes), then per symbol (f_s - 1) | c_s << 16 (256 words). Wave 0 forms
// the cumulative counts; then thread i fills slots [16 i, 16 i + 16) in LDS
// (one search for its first slot, then a walk), and the tables are copied
// out.
constexpr int kLzSlotsPer = (int)kLzM / kLzThreads;
__global__ void __launch_bounds__(kLzThreads) lz_dmodel_kernel(const LzArgs a) {
  __shared__ uint32_t cum[257];
  __shared__ uint32_t frq[256];
  __shared__ uint32_t total;
  __shared__ __align__(16) uint8_t tb[kLzM];
  const int ji = lz_job_at<&LzJob::field0>(a, blockIdx.x);
  const LzJob& j = a.jobs[ji];
  if (lz_failed(a, j)) return;
  const LzShape s = lz_shape(a, j);
  const int f = blockIdx.x - j.field0, tid = threadIdx.x;
  if (lz_n(s, f) == 0) return;
  const int A = lz_alpha(s, f);
  const LzField fd = lz_field(s, f);
  const LzLayout L = lz_layout(s, false);
  if (tid < 64) {
    const int lane = tid;
    const uint16_t* fr = (const uint16_t*)(j.src + fd.tab_off + 8);
    uint32_t run = 0;
    for (int q = 0; q < 4; ++q) {
      const int sy = lane + 64 * q;
      const uint32_t fv = sy < A ? fr[sy] : 0u;
      const uint32_t inc = wave_scan(fv, lane);
      cum[sy] = sy < A ? run + inc - fv : 0xFFFFFFFFu;
      frq[sy] = fv;
      run += (uint32_t)__shfl((int)inc, 63, 64);
    }
    if (lane == 0) {
      cum[256] = 0xFFFFFFFFu;
      total = run;
    }
  }
  __syncthreads();
  if (total != kLzM) {   // uniform
    if (tid == 0) lz_set(a, j, KVTC_E_CORRUPT);
    return;
  }
  const uint32_t s0 = (uint32_t)tid * kLzSlotsPer;
  int lo = 0, hi = A - 1;            // the last symbol whose range starts at or before s0
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cum[mid] <= s0) lo = mid;
    else hi = mid - 1;
  }
  uint32_t w[kLzSlotsPer / 4] = {};
#pragma unroll
  for (int i = 0; i < kLzSlotsPer; ++i) {
    while (cum[lo + 1] <= s0 + (uint32_t)i) ++lo;  // symbols without slots share the next one's start
    w[i / 4] |= (uint32_t)lo << (8 * (i % 4));
  }
  static_assert(kLzSlotsPer == 16, "one 16-byte store of slot symbols per thread");
  ((u32x4*)tb)[tid] = (u32x4){w[0], w[1], w[2], w[3]};
  __syncthreads();
  uint8_t* out = j.ws + L.aux + (size_t)f * kLzM * 4;
  for (int i = tid; i < (int)kLzM / 16; i += kLzThreads) ((u32x4*)out)[i] = ((const u32x4*)tb)[i];
  // symbols without slots (past the alphabet, or of count 0) get 0: no
  // slot names them
  ((uint32_t*)(out + kLzM))[tid] = tid < A && frq[tid] ? (frq[tid] - 1u) | (cum[tid] << 16) : 0u;
}

// One wavefront per chunk, lane l decoding symbols 64 t + l with its own
// state: per step the slot's symbol, its (f, c) and the state update, then the lanes
// whose state fell below L take the next words in lane order (ballot and
// prefix count). Everything the loop reads is in LDS: the two tables (5 KiB,
// so a workgroup holds 9 KiB and every chunk of a launch can be resident), and
// the payload in a ring of two 1 KiB blocks; the block after those is
// already loaded into registers and enters the ring when the ring's older
// block is used up, so each global load has about ten steps to arrive.
// Symbols are staged in LDS and stored 16 steps (1 KiB) at a time.
constexpr uint32_t kLzBlk = 1024;            // payload bytes per ring block (64 lanes x 16)
__global__ void __launch_bounds__(kLzLanes) lz_decode_kernel(const LzArgs a) {
  __shared__ __align__(16) uint8_t tsym[kLzM];
  __shared__ __align__(16) uint32_t tfc[256];
  __shared__ __align__(16) uint8_t syms[16 * kLzLanes];
  __shared__ __align__(16) uint8_t ring[2 * kLzBlk];
  const uint32_t g = blockIdx.x;
  const int l = threadIdx.x;
  const int ji = lz_job_at<&LzJob::chunk0>(a, g);
  const LzJob& j = a.jobs[ji];
  if (lz_failed(a, j)) return;
  const LzShape s = lz_shape(a, j);
  const uint32_t kj = g - j.chunk0;
  uint32_t k = kj, sym_off = 0;
  int f = 0;
  for (; f < lz_nf(s); ++f) {
    const uint32_t nc = lz_chunks(lz_n(s, f));
    if (k < nc) break;
    k -= nc;
    sym_off += lz_sym_region(lz_n(s, f));
  }
  const LzLayout L = lz_layout(s, false);
  const u32x4* gt = (const u32x4*)(j.ws + L.aux + (size_t)f * kLzM * 4);
  for (int i = l; i < (int)(kLzM + 1024) / 16; i += kLzLanes) {
    const u32x4 v = gt[i];
    if (i < (int)kLzM / 16) ((u32x4*)tsym)[i] = v;
    else ((u32x4*)tfc)[i - kLzM / 16] = v;
  }
  const uint32_t len = min((uint32_t)kLzChunk, lz_n(s, f) - k * kLzChunk);
  const int steps = (int)((len + kLzLanes - 1) / kLzLanes);
  const uint32_t* dir = (const uint32_t*)(j.src + L.dir_off);
  const uint32_t total = ((const uint32_t*)j.src)[6];
  const uint32_t start = L.pay_off + (kj ? dir[kj - 1] : 0u);
  const uint32_t nw = (L.pay_off + dir[kj] - start) / 2;     // >= 128, checked
  // blocks of the container from a0 = start rounded down to 16; byte
  // off0 + 2 p of block space is payload word p
  const uint32_t a0 = start & ~15u, off0 = start - a0;
  auto blk = [&](uint32_t b) -> u32x4 {
    const uint32_t at = a0 + b * kLzBlk + 16u * (uint32_t)l;
    return at < total ? *(const u32x4*)(j.src + at) : u32x4(0u);
  };
  const u32x4 b0 = blk(0), b1 = blk(1);
  u32x4 pend = blk(2);
  ((u32x4*)ring)[l] = b0;
  ((u32x4*)ring)[kLzLanes + l] = b1;
  __syncthreads();
  const uint16_t* rw = (const uint16_t*)ring;
  auto word = [&](uint32_t p) -> uint32_t { return rw[((off0 + 2 * p) & (2 * kLzBlk - 1)) >> 1]; };
  uint32_t x = word(2 * l) | (word(2 * l + 1) << 16);
  uint32_t pos = 2 * kLzLanes, cur = 0;
  u32x4* out = (u32x4*)(j.ws + sym_off + (size_t)k * kLzChunk);
  bool ok = true;
  for (int t = 0; t < steps; ++t) {
    const uint32_t i = (uint32_t)t * kLzLanes + l;
    const bool act = i < len;
    const uint32_t slot = x & (kLzM - 1);
    const uint32_t sy = tsym[slot];
    const uint32_t e = tfc[sy];
    if (act) x = ((e & 0xFFFFu) + 1u) * (x >> kLzMBits) + slot - (e >> 16);
    syms[(t & 15) * kLzLanes + l] = (uint8_t)sy;
    if ((t & 15) == 15 || t == steps - 1) {   // 16 steps staged: 1 KiB out, 16 bytes a lane
      const uint32_t q = (uint32_t)(t & ~15) * kLzLanes / 16 + l;
      if (q * 16 < len) out[q] = ((const u32x4*)syms)[l];
    }
    const bool need = act && x < kLzL;
    const uint64_t mask = __ballot(need);
    const uint32_t kn = (uint32_t)__popcll(mask);
    if (pos + kn > nw) {
      ok = false;
      break;
    }
    if (need) x = (x << 16) | word(pos + (uint32_t)__popcll(mask & lanes_below(l)));
    pos += kn;
    const uint32_t nb = (off0 + 2 * pos) / kLzBlk;
    if (nb > cur) {                   // block cur used up: its ring half takes block cur + 2
      ((u32x4*)ring)[(cur & 1) * kLzLanes + l] = pend;
      cur = nb;
      pend = blk(cur + 2);
    }
  }
  const bool bad = !ok || pos != nw || __ballot(x != kLzL) != 0ull;
  if (bad && l == 0) lz_set(a, j, KVTC_E_CORRUPT);
}

// One unit per block of passthrough elements or records: field symbols back
// into the stream (nothing is written for a job found bad). Unit 0 of a job
// also copies the stream header. A record block stages its symbols in LDS
// (8 planes of 64 n_act bytes, then n_act code runs of 64 G bytes); each
// thread assembles whole (record, group) items in registers, writes them
// into the packed records over the staged symbols, and the block leaves in
// 16-byte stores.
__global__ void __launch_bounds__(kLzThreads) lz_merge_kernel(const LzArgs a) {
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ uint32_t pcw_l[KVTC_MAX_REFF];
  const int ji = lz_job_at<&LzJob::unit0>(a, blockIdx.x);
  const LzJob& j = a.jobs[ji];
  if (lz_failed(a, j)) return;
  const LzShape s = lz_shape(a, j);
  const uint32_t u = blockIdx.x - j.unit0;
  const int tid = threadIdx.x;
  uint8_t* dst = j.dst;
  if (u == 0 && tid < 16) ((uint32_t*)dst)[tid] = ((const uint32_t*)(j.src + kLzHead))[tid];
  const uint32_t n_pb = (s.n_pt + kLzPassBlk - 1) / kLzPassBlk;
  const uint8_t* sym = j.ws;
  if (u < n_pb) {
    // 16 consecutive elements a thread: a 16-byte load per plane (the
    // regions are padded), 16-byte stores of the elements
    const uint32_t e0 = u * kLzPassBlk + 16 * tid;
    if (e0 >= s.n_pt) return;
    const uint32_t rp = lz_sym_region(s.n_pt);
    u32x4 pl[4];
    for (int b = 0; b < s.esz; ++b) pl[b] = *(const u32x4*)(sym + b * rp + e0);
    uint8_t* out = dst + kHeaderBytes + (size_t)e0 * s.esz;
    if (e0 + 16 <= s.n_pt) {
      for (int v = 0; v < s.esz; ++v) {
        u32x4 w;
        for (int q = 0; q < 4; ++q) {
          uint32_t x = 0;
          if (s.esz == 2) {
            const int e = 8 * v + 2 * q;
            const uint32_t lo = pl[0][e >> 2] >> (8 * (e & 3)), hi = pl[1][e >> 2] >> (8 * (e & 3));
            x = (lo & 0xFFu) | ((hi & 0xFFu) << 8) | ((lo & 0xFF00u) << 8) | ((hi & 0xFF00u) << 16);
          } else {
            const int e = 4 * v + q;
            for (int b = 0; b < 4; ++b) x |= ((pl[b][e >> 2] >> (8 * (e & 3))) & 0xFFu) << (8 * b);
          }
          w[q] = x;
        }
        ((u32x4*)out)[v] = w;
      }
    } else {
      for (uint32_t e = 0; e < s.n_pt - e0; ++e)
        for (int b = 0; b < s.esz; ++b) out[e * s.esz + b] = (uint8_t)(pl[b][e >> 2] >> (8 * (e & 3)));
    }
    return;
  }
  const uint32_t r0 = (u - n_pb) * kLzRecBlk;
  if (r0 >= s.tc) return;
  const DevSlot* sl = lz_slot(a, j);
  const int rb = sl->record_bytes, na = s.n_act, G = s.G;
  const int nr = (int)min((uint32_t)kLzRecBlk, s.tc - r0);
  // stage: planes at k * 64 na, codes of group g at 8 * 64 na + g * 64 G
  // (whole words; a word past a run's end reads padding or the next block)
  const int pl_b = kLzRecBlk * na, cd_b = kLzRecBlk * G;
  for (int k = 0; k < 8; ++k) {
    const uint32_t* in = (const uint32_t*)(sym + lz_plane_off(s, s.esz + k) + (size_t)r0 * na);
    for (int i = tid; i < (nr * na + 3) / 4; i += kLzThreads) ((uint32_t*)(lds + k * pl_b))[i] = in[i];
  }
  for (int g = 0; g < na; ++g) {
    const uint32_t* in = (const uint32_t*)(sym + lz_code_off(s, g) + (size_t)r0 * G);
    for (int i = tid; i < nr * G / 4; i += kLzThreads) ((uint32_t*)(lds + 8 * pl_b + g * cd_b))[i] = in[i];
  }
  // With a width per component, the slot's table ((record bit << 8) | width
  // per component of each active group) in LDS.
  const bool pc = sl->pc != 0;
  if (pc) {
    const uint32_t* pcw = (const uint32_t*)(a.state + sl->pcw_off);
    for (int i = tid; i < na * G; i += kLzThreads) pcw_l[i] = pcw[i];
  }
  __syncthreads();
  // Each thread assembles whole (record, group) items in registers: the 8
  // bytes of the group's (shift, scale) and its code chunk (each code at its
  // bit offset in the chunk, LSB first). At most 64 * 16 items per block
  // (KVTC_MAX_REFF components), so at most kLzItems per thread.
  constexpr int kLzItems = kLzRecBlk * (KVTC_MAX_REFF / 16) / kLzThreads;
  const int n_it = nr * na;
  uint32_t ssw[kLzItems][2];
  uint64_t acc[kLzItems][4];
#pragma unroll
  for (int k = 0; k < kLzItems; ++k) {
    const int it = tid + kLzThreads * k;
    ssw[k][0] = ssw[k][1] = 0u;
    acc[k][0] = acc[k][1] = acc[k][2] = acc[k][3] = 0ull;
    if (it >= n_it) continue;
    const int t = it / na, g = it - t * na;
#pragma unroll
    for (int q = 0; q < 8; ++q) ssw[k][q >> 2] |= (uint32_t)lds[q * pl_b + t * na + g] << (8 * (q & 3));
    const uint8_t* cq = lds + 8 * pl_b + g * cd_b + t * G;
    const int b = s.width[g];
    for (int c = 0; c < G; ++c) {
      int rel = c * b, w = b;
      if (pc) {
        const uint32_t e = pcw_l[g * G + c];
        rel = (int)(e >> 8) - 8 * sl->chunk_off[g];
        w = (int)(e & 0xFFu);
      }
      const uint64_t qv = (uint64_t)(cq[c] & ((1u << w) - 1u));
      const int wi = rel >> 6, sh = rel & 63;
      // a code never crosses two words' boundary by more than its 8 bits
      uint64_t lo = qv << sh, hi = sh ? qv >> (64 - sh) : 0ull;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        if (x == wi) acc[k][x] |= lo;
        if (x == wi + 1) acc[k][x] |= hi;
      }
    }
  }
  __syncthreads();   // every staged symbol is read
  // The block's records, packed, over the staged symbols (they take at most
  // the same bytes: rb <= na * (8 + G)).
#pragma unroll
  for (int k = 0; k < kLzItems; ++k) {
    const int it = tid + kLzThreads * k;
    if (it >= n_it) continue;
    const int t = it / na, g = it - t * na;
    uint8_t* rw = lds + t * rb;
#pragma unroll
    for (int q = 0; q < 8; ++q) rw[8 * g + q] = (uint8_t)(ssw[k][q >> 2] >> (8 * (q & 3)));
    const int co = sl->chunk_off[g];
    const int cb = (g + 1 < na ? sl->chunk_off[g + 1] : rb) - co;   // the chunk's bytes
    for (int y = 0; y < cb; ++y) {
      uint64_t wv = 0;
#pragma unroll
      for (int x = 0; x < 4; ++x)
        if (x == (y >> 3)) wv = acc[k][x];
      rw[co + y] = (uint8_t)(wv >> (8 * (y & 7)));
    }
  }
  __syncthreads();
  uint8_t* base = dst + kHeaderBytes + (size_t)s.n_pt * s.esz + (size_t)r0 * rb;
  const int nbytes = nr * rb;
  // 16-byte copies (base is 16-byte aligned: the header, n_pt * esz and
  // 64 * rb are multiples of 16), then the tail
  for (int v = tid; v < nbytes / 16; v += kLzThreads) ((u32x4*)base)[v] = ((const u32x4*)lds)[v];
  for (int y = (nbytes & ~15) + tid; y < nbytes; y += kLzThreads) base[y] = lds[y];
}

}  // namespace

int launch_lz_encode(const LzArgs& a, hipStream_t s) {
  if (a.units) hipLaunchKernelGGL(lz_split_kernel, dim3(a.units), dim3(kLzThreads), a.rec_lds, s, a);
  if (a.segs) hipLaunchKernelGGL(lz_hist_kernel, dim3(a.segs), dim3(kLzThreads), 0, s, a);
  if (a.fields) hipLaunchKernelGGL(lz_model_kernel, dim3(a.fields), dim3(64), 0, s, a);
  if (a.chunks) hipLaunchKernelGGL(lz_code_kernel, dim3(a.chunks), dim3(kLzLanes), 0, s, a);
  hipLaunchKernelGGL(lz_layout_kernel, dim3(a.n_jobs), dim3(kLzThreads), 0, s, a);
  if (a.chunks) hipLaunchKernelGGL(lz_copy_kernel, dim3(a.chunks), dim3(kLzThreads), 0, s, a);
  return (int)hipGetLastError();
}

int launch_lz_decode(const LzArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(lz_check_kernel, dim3(a.n_jobs), dim3(kLzThreads), 0, s, a);
  if (a.fields) hipLaunchKernelGGL(lz_dmodel_kernel, dim3(a.fields), dim3(kLzThreads), 0, s, a);
  if (a.chunks) hipLaunchKernelGGL(lz_decode_kernel, dim3(a.chunks), dim3(kLzLanes), 0, s, a);
  if (a.units) hipLaunchKernelGGL(lz_merge_kernel, dim3(a.units), dim3(kLzThreads), a.rec_lds, s, a);
  return (int)hipGetLastError();
}

}  // namespace kvtc
