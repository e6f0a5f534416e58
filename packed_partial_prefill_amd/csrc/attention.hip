// Packed causal attention over the mixed cache with the metadata bias.
//
// Query row r (position u = T[r]), head h reads KV head g = h / (Hq/Hkv)
// over keys j = 0..u inclusive ("Budgeted KV-Cache Repair", section 13.2,
// Eq. 22) with logits <q, k_j>/sqrt(d) + alpha*[local_j] + beta*[sink_j]
// (cross-attention reuse page, 6.4) and an online softmax.
//
// bf16 storage runs on MFMA kernels followed by a merge kernel: k_attn_pp
// (d = 128, launches with many KV tiles per CU: two query tiles per
// workgroup in ping-pong phases, stream-K schedule) or k_attn_mfma (d = 64
// and small launches: one query tile per workgroup, split-KV); float32
// storage runs on a VALU kernel: one wave per (row, head), each 64-key step
// scores one key per lane, then accumulates P*V with every lane owning d/64
// output columns.
#include <type_traits>

#include "common.h"
#include "kvr_internal.h"

namespace kvr {

namespace {

template <typename T>
__global__ __launch_bounds__(64) void k_attn_rowwise(const T* __restrict__ q,
                                                     const T* __restrict__ kc,
                                                     const T* __restrict__ vc,
                                                     const uint8_t* __restrict__ flags,
                                                     const int32_t* __restrict__ Tpos, Shape sh,
                                                     float alpha, float beta, T* __restrict__ o) {
  __shared__ float qs[128];
  __shared__ float ps[64];
  const int r = blockIdx.x / sh.hq, h = blockIdx.x - r * sh.hq;
  const int g = h / sh.group;
  const int u = Tpos[r];
  const int d = sh.d, lane = threadIdx.x;
  const int per = d >> 6;  // 1 or 2 output columns per lane
  const T* qr = q + (static_cast<size_t>(r) * sh.hq + h) * d;
  for (int c = lane; c < d; c += 64) qs[c] = Elem<T>::load(qr, c);
  __syncthreads();
  const float scale = rsqrtf(static_cast<float>(d));
  const size_t kv_stride = static_cast<size_t>(sh.hkv) * d;
  float m = -INFINITY, l = 0.f, acc[2] = {0.f, 0.f};
  for (int j0 = 0; j0 <= u; j0 += 64) {
    const int j = j0 + lane;
    float s = -INFINITY;
    if (j <= u) {
      const T* kr = kc + j * kv_stride + static_cast<size_t>(g) * d;
      float dot = 0.f;
      for (int c = 0; c < d; ++c) dot = fmaf(qs[c], Elem<T>::load(kr, c), dot);
      const uint8_t f = flags[j];
      s = dot * scale + ((f & KVR_FLAG_LOCAL) ? alpha : 0.f) + ((f & KVR_FLAG_SINK) ? beta : 0.f);
    }
    const float mn = fmaxf(m, wave_max(s));
    const float p = (j <= u) ? expf(s - mn) : 0.f;
    const float corr = expf(m - mn);
    l = l * corr + wave_sum(p);
    ps[lane] = p;
    __syncthreads();
    acc[0] *= corr;
    acc[1] *= corr;
    const int nk = min(64, u + 1 - j0);
    for (int jj = 0; jj < nk; ++jj) {
      const float pj = ps[jj];
      const T* vr = vc + (j0 + jj) * kv_stride + static_cast<size_t>(g) * d;
      for (int c = 0; c < per; ++c) acc[c] = fmaf(pj, Elem<T>::load(vr, lane * per + c), acc[c]);
    }
    m = mn;
    __syncthreads();
  }
  T* orow = o + (static_cast<size_t>(r) * sh.hq + h) * d;
  const float inv = 1.f / l;
  for (int c = 0; c < per; ++c) Elem<T>::store(orow, lane * per + c, acc[c] * inv);
}

// ---------------------------------------------------------------------------
// bf16 MFMA kernel (gfx950 v_mfma_f32_32x32x16_bf16), float32 softmax.
//
// A workgroup owns KVR_ATTN_QROWS = 128 (packed row, query head) pairs of one
// KV head group and a range of 64-key tiles (split-KV), 32 pairs per wave.
// Every key tile is staged once in LDS for all the workgroup's pairs by
// global_load_lds_dwordx4 (no register staging), with its 64 flag bytes, in
// kAttnStages buffers (the tile in use and the ones in flight).  With 128
// pairs, two workgroups share a CU in two stages each, so one computes while
// the other waits at its barrier; 256 pairs per workgroup without phase
// offsets (half the staging bytes per MFMA, three stages, one workgroup per
// CU) measured slower: both waves of a SIMD then compute and exponentiate at
// the same time (k_attn_pp below offsets them).  K and V are both in their
// natural [key][d] layout with the 16-byte chunks of each key row
// XOR-swizzled, and the tile's flag bytes give each key's bias slice.
// Scores are formed transposed, S^T = K Q^T, so each lane owns one query
// column and 16 of the tile's keys: the softmax reduction is in-lane plus one
// exchange with lane ^ 32.  O^T += V^T P^T takes the lane's own P values as
// the B operand; its A operand (V^T rows) comes from ds_read_b64_tr_b16,
// which hands each lane 4 keys of one d column out of 16 lanes' row reads.
// Both operands list the keys of a 16-key step in the same order (4h..4h+3,
// 8+4h..8+4h+3 for lane half h).
// Tiles below the plan's n_full (Eq. 23) are visible to every pair and skip
// the causal test.  Q arrives pre-scaled by log2(e)/sqrt(d), so the softmax
// runs in base 2 with the bias pre-multiplied by log2(e); bias and running
// maximum enter through the score MFMA, leaving max, exp2, sum and the bf16
// pack as the per-score VALU work.
// ---------------------------------------------------------------------------
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef short s16x4_t __attribute__((ext_vector_type(4)));

constexpr int kQRows = KVR_ATTN_QROWS;     // 128 pairs per workgroup
constexpr int kKvTile = KVR_ATTN_KV_TILE;  // 64 keys per tile
constexpr int kAttnThreads = 256;          // merge and decode kernels
constexpr int kAttnWaves = kQRows / 32;    // packed kernel: 32 pairs per wave
constexpr int kAttnMfmaThreads = 64 * kAttnWaves;
constexpr int kAttnWgPerCu = 8 / kAttnWaves;   // 8 waves per CU (2 per SIMD)
// KV tiles in LDS: the current one plus kAttnStages - 1 in flight (three
// stages fit one 256-pair workgroup per CU, two stages two 128-pair ones)
constexpr int kAttnStages = kAttnWgPerCu == 1 ? 3 : 2;

#define KVR_LDS(p) ((__attribute__((address_space(3))) void*)(p))
#define KVR_GLB(p) ((const __attribute__((address_space(1))) void*)(p))

template <int N> __device__ __forceinline__ void attn_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0xF70);
}

// Global loads the compiler does not know of: the caller waits for them
// (vmcnt, issue order) and fences their registers before the first use.
__device__ __forceinline__ u32x4_t untracked_load_b128(const void* p) {
  u32x4_t r;
  asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(r) : "v"(p) : "memory");
  return r;
}
__device__ __forceinline__ uint32_t untracked_load_b32(const void* p) {
  uint32_t r;
  asm volatile("global_load_dword %0, %1, off" : "=v"(r) : "v"(p) : "memory");
  return r;
}

template <int D>
struct AttnLds {
  static constexpr int kBytes = kKvTile * D * 2;   // K tile
  static constexpr int vBytes = kKvTile * D * 2;   // V tile
  static constexpr int fBytes = kKvTile;           // the tile's metadata flag bytes
  static constexpr int stage = kBytes + vBytes + fBytes;
  static constexpr int total = kAttnStages * stage;
  // Regions by operand (K of every stage, then V, then the flags), so that
  // every address within a region is a lane register plus an immediate
  // offset below 64 KB.
  static constexpr int kOff(int b) { return b * kBytes; }
  static constexpr int vOff(int b) { return kAttnStages * kBytes + b * vBytes; }
  static constexpr int fOff(int b) { return kAttnStages * (kBytes + vBytes) + b * fBytes; }
  static constexpr int slices = (kBytes + vBytes) / 1024 / kAttnWaves;   // 1 KB DMA slices per wave
  static_assert((kBytes + vBytes) % (1024 * kAttnWaves) == 0, "DMA slices per wave");
};

// Physical 16-byte chunk of logical chunk c in key row k.  K rows: c ^ (k & 15)
// (d = 128) or c ^ ((k & 7) ^ ((k >> 3) & 1)) (d = 64), so the 32 rows of an
// MFMA operand read hit distinct bank slots.  V rows (d = 128): c ^ (4 (k & 3)),
// which measures no bank conflicts for the transposing reads on gfx950
// (rocprofv3 SQ_LDS_BANK_CONFLICT; c ^ (2 (k & 3)) measured 2-way); d = 64
// keeps c ^ (2 (k & 3)) within its 8 chunks.
template <int D>
__device__ __forceinline__ int kchunk(int key, int c) {
  return c ^ ((D == 128) ? (key & 15) : ((key & 7) ^ ((key >> 3) & 1)));
}
template <int D>
__device__ __forceinline__ int vchunk(int key, int c) {
  return c ^ ((D == 128) ? ((key & 3) << 2) : (2 * (key & 3)));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// ds_read_b64_tr_b16 at LDS byte address addr + OFF.  Written as inline
// assembly because the compiler places a wait for every outstanding LDS DMA
// in front of the builtin form (it cannot tell that the DMA in flight
// targets another buffer), which would stall each tile on the prefetch of
// the next.  The caller waits for the result with lds_wait().
template <int OFF>
__device__ __forceinline__ u32x2_t ds_read_tr16(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
  u32x2_t r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF) : "memory");
  return r;
}
// ds_read_u8 at addr + OFF (see ds_read_tr16 for why assembly).
template <int OFF>
__device__ __forceinline__ uint32_t ds_read_u8(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
  uint32_t r;
  asm volatile("ds_read_u8 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF) : "memory");
  return r;
}

// Workgroup barrier for the KV pipeline.  __syncthreads() (and any
// workgroup release fence, since LDS DMA writes count as LDS stores) waits
// for every outstanding global load, which would drain the KV tiles still in
// flight.  Here each wave waits for its own LDS reads and writes
// (lgkmcnt 0) and for the DMA of the next tile (attn_wait_vmcnt, before the
// call); the empty asm statements keep the compiler from moving LDS
// accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  lds_wait();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int D>
__global__ __launch_bounds__(kAttnMfmaThreads, kAttnWgPerCu) void k_attn_mfma(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ kc, const bf16_t* __restrict__ vc,
    const uint8_t* __restrict__ flags, const int32_t* __restrict__ Tpos,
    const int32_t* __restrict__ n_full, const int32_t* __restrict__ n_total, int B, int n_tokens,
    int Hq, int Hkv, int G, float bias_local, float bias_sink, int split_tiles, int n_splits,
    float* __restrict__ part_o, float* __restrict__ part_ml) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  using L = AttnLds<D>;
  constexpr int KCH = D / 8;             // 16-byte chunks per key row
  constexpr int ROWS = 1024 / (D * 2);   // key rows per 1 KB DMA slice
  // Plain block order (query tile fastest): every XCD takes every KV range.
  // Grouping the query tiles of one KV range on one XCD (by split, or by a
  // fixed residue class of (head, split)) measured 33-37% slower.
  const int qt = blockIdx.x, g = blockIdx.y, sp = blockIdx.z;
  const int tot = n_total[qt];
  const int c0 = sp * split_tiles;
  if (c0 >= tot) return;
  const int c1 = min(tot, c0 + split_tiles);
  const int nf = n_full[qt];
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int P = B * G;

  // the query column this lane owns
  const int p = qt * kQRows + wave * 32 + (lane & 31);
  const int pc = min(p, P - 1);
  const int r = pc / G;
  const int h = g * G + (pc - r * G);
  const int u = Tpos[r];
  bf16x8_t qf[D / 16];
  {
    const bf16_t* qrow = q + (static_cast<size_t>(r) * Hq + h) * D + 8 * half;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qf[ks] = *reinterpret_cast<const bf16x8_t*>(qrow + ks * 16);
  }
  // the query fragments have arrived before the loop (otherwise the wait for
  // them would sit inside it, in front of every tile's first product)
  attn_wait_vmcnt<0>();
  // The score MFMA takes one more 16-wide K slice: key j supplies
  // [b_hi, b_lo, 1, 1, 0...] (b_hi + b_lo = bf16 split of the key's bias),
  // the query supplies [1, 1, -m_hi, -m_lo, 0...] (lanes of the upper half
  // supply zeros), so the MFMA yields s + bias - m_eff with
  // m_eff = m_hi + m_lo the query's current reference maximum.
  float m_eff = 0.f;
  bool m_set = false;
  bf16x8_t qx;
  auto set_qx = [&](float mref) {
    const bf16_t mh = f32_to_bf16(-mref);
    const bf16_t ml = f32_to_bf16(-mref - bf16_to_f32(mh));
    m_eff = -(bf16_to_f32(mh) + bf16_to_f32(ml));
    const bf16_t one = 0x3F80;
    const bf16_t v[8] = {one, one, mh, ml, 0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 8; ++i) qx[i] = __builtin_bit_cast(__bf16, half == 0 ? v[i] : static_cast<bf16_t>(0));
  };
  set_qx(0.f);

  const size_t kv_row = static_cast<size_t>(Hkv) * D;   // elements between positions
  const bf16_t* kg = kc + static_cast<size_t>(g) * D;
  const bf16_t* vg = vc + static_cast<size_t>(g) * D;

  // DMA slices of this wave: slice j covers key rows [j*ROWS, (j+1)*ROWS) of
  // K (j < 64/ROWS) or V.  Lane i lands at byte i*16 of the slice: row
  // i / KCH, physical chunk i % KCH, so it fetches the matching logical chunk.
  // A tile's source is a wave-uniform base (its first key row of K or V) plus
  // this lane's loop-invariant 32-bit byte offset.
  constexpr int KSL = kKvTile / ROWS;   // slices per operand per tile (16 or 8)
  const size_t row_bytes = kv_row * 2;
  // slice j of this wave: operand (wave-uniform) and this lane's byte offset
  // within the tile (key row, logical 16-byte chunk)
  auto slice_isv = [&](int j) { return wave * L::slices + j >= KSL; };
  uint32_t s_off[L::slices];
  int s_dst[L::slices];
#pragma unroll
  for (int j = 0; j < L::slices; ++j) {
    const int sl = wave * L::slices + j;         // wave-uniform
    const int row = (sl >= KSL ? sl - KSL : sl) * ROWS + lane / KCH, phys = lane % KCH;
    const int logical = slice_isv(j) ? vchunk<D>(row, phys) : kchunk<D>(row, phys);   // involutions
    s_off[j] = static_cast<uint32_t>(row * row_bytes) + logical * 16;
    s_dst[j] = (slice_isv(j) ? L::vOff(0) : L::kOff(0)) + (sl >= KSL ? sl - KSL : sl) * 1024;
  }
  const uint8_t* kg8 = reinterpret_cast<const uint8_t*>(kg);
  const uint8_t* vg8 = reinterpret_cast<const uint8_t*>(vg);
  static_assert(L::kBytes == L::vBytes, "K and V stages advance by the same stride");
  // Tile c into buffer BUF by buffer loads into LDS: per tile a wave-uniform
  // descriptor whose range is the tile's rows inside the cache (rows past
  // the cache read as zero; those keys are always masked), each lane a 32-bit
  // offset.  Wave 0 also brings the 64 flag bytes, 4 per lane, issued first;
  // the last, partial tile stages its flags through registers instead (a
  // range-checked dword straddling the end would read as zero), and a
  // compiler wait then drains everything issued before.  A wave issues
  // L::slices (+1 on wave 0) vector-memory operations per full tile.
  constexpr int kRsrcWord3 = 0x00020000;   // raw (untyped) buffer access
  auto issue = [&](int c, auto bufc) {
    constexpr int BUF = decltype(bufc)::value;
    const int kv0 = c * kKvTile;
    const int rows = min(kKvTile, n_tokens - kv0);
    const int nbytes = rows * static_cast<int>(row_bytes);
    if (wave == 0) {
      if (rows == kKvTile) {
        if (lane < kKvTile / 4) {
          const __amdgpu_buffer_rsrc_t rf = __builtin_amdgcn_make_buffer_rsrc(
              const_cast<uint8_t*>(flags + kv0), 0, kKvTile, kRsrcWord3);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rf, KVR_LDS(lds + L::fOff(BUF)), 4, 4 * lane, 0,
                                                   0, 0);
        }
      } else {
        lds[L::fOff(BUF) + lane] = flags[min(kv0 + lane, n_tokens - 1)];
      }
    }
    // (descriptors are built per slice from the chosen base, and the lane
    // offset goes in as int: a conditional between descriptors, or an
    // unsigned offset argument, makes the host compilation pass silently
    // drop the kernel)
#pragma unroll
    for (int j = 0; j < L::slices; ++j) {
      const uint8_t* base = (slice_isv(j) ? vg8 : kg8) + static_cast<size_t>(kv0) * row_bytes;
      const __amdgpu_buffer_rsrc_t r =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0, nbytes, kRsrcWord3);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, KVR_LDS(lds + BUF * L::kBytes + s_dst[j]), 16,
                                               static_cast<int>(s_off[j]), 0, 0, 0);
    }
  };
  // this wave's part of tile c + 1 has landed, at the end of tile c, with
  // the tiles after it (kAttnStages - 2 of them) still in flight
  auto wait_next = [&]() {
    if (wave == 0)
      attn_wait_vmcnt<(kAttnStages - 2) * (L::slices + 1)>();
    else
      attn_wait_vmcnt<(kAttnStages - 2) * L::slices>();
  };

  // Score-MFMA operands.  K rows: key sb*32 + (lane % 32), 16-byte chunk
  // 2 ks + half; its swizzle depends on key % 16 only, so klane[ks] plus an
  // immediate (buffer, sb) addresses it.  Bias slice: key j supplies
  // [b_hi, b_lo, 1, 1, 0 x 4] (lanes of the upper half supply zeros), picked
  // from the four flag combinations by the key's flag byte.
  uint32_t klane[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
    klane[ks] = lds_addr(lds) + L::kOff(0) + (lane & 31) * (D * 2) +
                (kchunk<D>(lane & 31, ks * 2 + half) << 4);
  const uint32_t flane = lds_addr(lds) + L::fOff(0) + (lane & 31);
  auto bias_word = [&](float b) {
    const bf16_t bh = f32_to_bf16(b);
    const bf16_t bl = f32_to_bf16(b - bf16_to_f32(bh));
    return half == 0 ? (static_cast<uint32_t>(bh) | (static_cast<uint32_t>(bl) << 16)) : 0u;
  };
  const uint32_t bw_l = bias_word(bias_local), bw_s = bias_word(bias_sink);
  const uint32_t bw_ls = bias_word(bias_local + bias_sink);
  const uint32_t bones = half == 0 ? 0x3F803F80u : 0u;   // bf16 1.0, 1.0 times -m_hi, -m_lo
  auto bias_operand = [&](uint32_t f) {
    const uint32_t wl = (f & KVR_FLAG_SINK) ? bw_ls : bw_l;
    const uint32_t wn = (f & KVR_FLAG_SINK) ? bw_s : 0u;
    const uint32_t w = (f & KVR_FLAG_LOCAL) ? wl : wn;
    const u32x4_t v = {w, bones, 0u, 0u};
    return __builtin_bit_cast(bf16x8_t, v);
  };

  // transposing-read address pattern of this lane (see header comment)
  const int tr_key = (lane & 15) >> 2;                          // key within the 4-key group
  const int tr_d = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);    // d offset within a 32-row block
  // Transposing-read address of key (16-key step base) + key_l, column block
  // db: the V swizzle depends only on key % 4 = tr_key, so it is this lane's
  // loop-invariant vlane[db] plus the step base times the row size (an
  // immediate) plus the buffer's offset.
  uint32_t vlane[D / 32];
  {
    const int key_l = 4 * half + tr_key;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int d = db * 32 + tr_d;
      vlane[db] = lds_addr(lds) + L::vOff(0) + key_l * (D * 2) + (vchunk<D>(key_l, d >> 3) << 4) +
                  (d & 7) * 2;
    }
  }

  f32x16_t o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int t = 0; t < 16; ++t) o[db][t] = 0.f;
  float l = 0.f;

  // One key tile from buffer BUF, prefetching tile c + kAttnStages - 1 into
  // the buffer tile c - 1 used.  All LDS reads of the loop are issued as
  // inline assembly with explicit lgkmcnt waits: the compiler cannot tell
  // them from the LDS DMA in flight (to another buffer) and would otherwise
  // wait for that DMA before the first read.
  auto tile = [&](auto bufc, int c) {
    constexpr int BUF = decltype(bufc)::value;
    constexpr int NXT = (BUF + kAttnStages - 1) % kAttnStages;
    const bool ahead = c + kAttnStages - 1 < c1;
    if (ahead) issue(c + kAttnStages - 1, std::integral_constant<int, NXT>{});

    // S^T = K Q^T + (bias - m_eff) for the two 32-key halves of the tile.
    // The K fragments come in groups of KG 16-wide K slices, each group read
    // while the previous group's products run (two register buffers).
    constexpr int KG = 4, GPS = D / 16 / KG, NG = 2 * GPS;   // groups per half, in all
    f32x16_t s[2];
    uint32_t fb[2];
    fb[0] = ds_read_u8<BUF * L::fBytes>(flane);
    fb[1] = ds_read_u8<BUF * L::fBytes + 32>(flane);
    u32x4_t kb[2][KG];
    auto kread = [&](auto gic, u32x4_t(&dst)[KG]) {
      constexpr int gi = decltype(gic)::value, sb = gi / GPS, kq = gi % GPS;
      static_for<0, KG>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        dst[j] = ds_read_b128<L::kOff(BUF) + sb * 32 * D * 2>(klane[kq * KG + j]);
      });
    };
    kread(std::integral_constant<int, 0>{}, kb[0]);
    static_for<0, NG>([&](auto gic) {
      constexpr int gi = decltype(gic)::value, sb = gi / GPS, kq = gi % GPS;
      if constexpr (gi + 1 < NG) {
        kread(std::integral_constant<int, gi + 1>{}, kb[(gi + 1) & 1]);
        lds_wait_n<KG>();   // this group (and the flag bytes) landed
      } else {
        lds_wait();
      }
#pragma unroll
      for (int j = 0; j < KG; ++j) reg_fence(kb[gi & 1][j]);
      if constexpr (gi == 0) {
        reg_fence(fb[0]);
        reg_fence(fb[1]);
      }
      if constexpr (kq == 0) {
#pragma unroll
        for (int t = 0; t < 16; ++t) s[sb][t] = 0.f;
      }
#pragma unroll
      for (int j = 0; j < KG; ++j)
        s[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kb[gi & 1][j]),
                                                         qf[kq * KG + j], s[sb], 0, 0, 0);
      if constexpr (kq == GPS - 1)
        s[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bias_operand(fb[sb]), qx, s[sb], 0, 0, 0);
      // keep this group's products ahead of the next group's wait (the
      // scheduler would otherwise sink them past it)
      __builtin_amdgcn_sched_barrier(0);
    });
    // V^T operands of the first 16-key step, read while the softmax runs
    u32x2_t xv[2][D / 32][2];
    auto vread = [&](auto stc, u32x2_t(&dst)[D / 32][2]) {
      constexpr int st = decltype(stc)::value, sb = st / 2, hs = st % 2;
      constexpr int off = BUF * L::vBytes + (sb * 32 + hs * 16) * D * 2;
      static_for<0, D / 32>([&](auto dbc) {
        constexpr int db = decltype(dbc)::value;
        dst[db][0] = ds_read_tr16<off>(vlane[db]);
        dst[db][1] = ds_read_tr16<off + 8 * D * 2>(vlane[db]);
      });
    };
    vread(std::integral_constant<int, 0>{}, xv[0]);
    // causal test only on partially visible tiles (uniform branch)
    if (c >= nf) {
      const int lim = u - c * kKvTile;   // keys kl > lim lie in the future
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          const int kl = sb * 32 + 8 * (t >> 2) + 4 * half + (t & 3);
          if (kl > lim) s[sb][t] = -INFINITY;
        }
    }
    // tile maximum of s + bias - m_eff, as a tree (a chain of 16 dependent
    // max3 instructions sat on the critical path)
    float mx[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      mx[i] = fmaxf(fmaxf(s[i >> 2][4 * (i & 3)], s[i >> 2][4 * (i & 3) + 1]),
                    fmaxf(s[i >> 2][4 * (i & 3) + 2], s[i >> 2][4 * (i & 3) + 3]));
    float mt = fmaxf(fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3])),
                     fmaxf(fmaxf(mx[4], mx[5]), fmaxf(mx[6], mx[7])));
    mt = xor32_max(mt);
    // Lazy maximum: m_eff moves only when the tile exceeds it by more than 8
    // (log2 units) or is the query's first visible tile, so probabilities
    // stay below 2^8 and most tiles skip rescaling.  After a move the tile's
    // scores are re-based by the shift (only in waves where a lane moved).
    const bool bump = (mt > 8.f) || (!m_set && mt != -INFINITY);
    if (__builtin_amdgcn_ballot_w64(bump) != 0) {
      float shift = 0.f;
      if (bump) {
        const float old = m_eff;
        set_qx(m_eff + mt);
        shift = m_eff - old;
        const float corr = m_set ? fast_exp2(-shift) : 0.f;
        l *= corr;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int t = 0; t < 16; ++t) o[db][t] *= corr;
        m_set = true;
      }
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int t = 0; t < 16; ++t) s[sb][t] -= shift;
    }

#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int t = 0; t < 16; ++t) s[sb][t] = fast_exp2(s[sb][t]);
    // the tile's sum of P as a pairwise tree (not a chain of 32 dependent adds)
    {
      float ps[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) ps[i] = s[i >> 3][2 * (i & 7)] + s[i >> 3][2 * (i & 7) + 1];
#pragma unroll
      for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
        for (int i = 0; i < w; ++i) ps[i] = ps[i] + ps[i + w];
      l += ps[0];
    }

    // O^T += V^T P^T, four 16-key steps.  Step st + 1's operands are read
    // once step st's first column block has landed (at most 14 LDS reads
    // outstanding), and each block's product waits only for its own reads.
    static_for<0, 4>([&](auto stc) {
      constexpr int st = decltype(stc)::value, sb = st / 2, hs = st % 2;
      constexpr int NB = D / 32, NEXT = st + 1 < 4 ? 2 * NB : 0;
      auto& x = xv[st & 1];
      lds_wait_n<2 * (NB - 1)>();
      reg_fence(x[0][0]);
      reg_fence(x[0][1]);
      if constexpr (st + 1 < 4) vread(std::integral_constant<int, st + 1>{}, xv[(st + 1) & 1]);
      bf16x8_t pb;
#pragma unroll
      for (int i = 0; i < 8; ++i) pb[i] = static_cast<__bf16>(s[sb][hs * 8 + i]);
      static_for<0, NB>([&](auto dbc) {
        constexpr int db = decltype(dbc)::value;
        if constexpr (db > 0) {
          lds_wait_n<2 * (NB - 1 - db) + NEXT>();
          reg_fence(x[db][0]);
          reg_fence(x[db][1]);
        }
        const u32x4_t w = {x[db][0][0], x[db][0][1], x[db][1][0], x[db][1][1]};
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, w), pb,
                                                         o[db], 0, 0, 0);
      });
    });

    if (ahead && kAttnStages > 2)
      wait_next();   // tile c + 1 has landed (this wave's part)
    else
      attn_wait_vmcnt<0>();
    lds_barrier();
  };

  static_assert(kAttnStages == 2 || kAttnStages == 3, "pipeline depth");
  issue(c0, std::integral_constant<int, 0>{});
  if constexpr (kAttnStages == 3) {
    if (c0 + 1 < c1) {
      issue(c0 + 1, std::integral_constant<int, 1>{});
      wait_next();   // tile c0 has landed
    } else {
      attn_wait_vmcnt<0>();
    }
  } else {
    attn_wait_vmcnt<0>();
  }
  lds_barrier();
  for (int c = c0; c < c1; c += kAttnStages) {
    static_for<0, kAttnStages>([&](auto bc) {
      if (c + decltype(bc)::value < c1) tile(bc, c + decltype(bc)::value);
    });
  }

  // partial results: O^T columns (unnormalised), running max and sum
  const size_t slot = (static_cast<size_t>(qt) * Hkv + g) * n_splits + sp;
  const int ql = wave * 32 + (lane & 31);
  float* po = part_o + slot * D * kQRows;
  if (p < P) {   // columns past the last pair are never merged
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const int d = db * 32 + 8 * (t >> 2) + 4 * half + (t & 3);
        po[d * kQRows + ql] = o[db][t];
      }
  }
  l = xor32_add(l);
  if (half == 0 && p < P) {
    float* pm = part_ml + slot * 2 * kQRows;
    pm[ql] = m_set ? m_eff : -INFINITY;
    pm[kQRows + ql] = l;
  }
}

// ---------------------------------------------------------------------------
// Ping-pong form of the packed kernel (d = 128).  One workgroup of 8 waves
// takes two neighbouring 128-pair query tiles of one KV group, so every KV
// tile is staged in LDS once for 256 pairs.  Waves 0-3 (group A, the first
// query tile) and 4-7 (group B, the second) share SIMDs pairwise and run the
// same per-tile program one phase apart: a product phase (PV of the previous
// tile, then the scores of this one) and a softmax phase.  Phases end at
// workgroup barriers, so on every SIMD one wave's matrix products overlap the
// other wave's softmax.  Per wave the arithmetic, and its order, is that of
// k_attn_mfma.  Four LDS stages: tile i is read in phases 2i .. 2i+3 (scores,
// then PV, each by both groups), and tile i + 2 is issued at phase 2i, four
// phases before its first read.
constexpr int kPPWaves = 8;
constexpr int kPPThreads = 64 * kPPWaves;
constexpr int kPPStages = 4;
// stream-K ranges in XCD-contiguous runs (neighbouring pieces share KV tiles)
constexpr bool kAttnXcdOrder = true;
// fewest KV tiles per stream-K workgroup (small problems use fewer CUs
// rather than paying a piece's prologue and epilogue for one or two tiles)
constexpr int kSkMinTiles = 4;
// cost of a piece's prologue and epilogue in KV tiles, charged per segment in
// the stream-K split (a workgroup with an extra piece takes fewer tiles)
constexpr int kSkPieceCost = 3;

template <int D>
struct PPLds {
  static constexpr int kBytes = kKvTile * D * 2;
  static constexpr int vBytes = kKvTile * D * 2;
  static constexpr int fBytes = kKvTile;
  static constexpr int total = kPPStages * (kBytes + vBytes + fBytes);
  static constexpr int kOff(int b) { return b * kBytes; }
  static constexpr int vOff(int b) { return kPPStages * kBytes + b * vBytes; }
  static constexpr int fOff(int b) { return kPPStages * (kBytes + vBytes) + b * fBytes; }
  static constexpr int slices = (kBytes + vBytes) / 1024 / kPPWaves;
  static_assert((kBytes + vBytes) % (1024 * kPPWaves) == 0, "DMA slices per wave");
  // immediate offsets: K reads up to kOff(3) + 32 rows, V reads (relative to
  // vOff(0)) up to 3 stages + 64 rows
  static_assert(kOff(kPPStages - 1) + kBytes <= 65536 && (kPPStages - 1) * vBytes + vBytes <= 65536,
                "ds offset field");
};

template <int D>
__global__ __launch_bounds__(kPPThreads, 1) void k_attn_pp(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ kc, const bf16_t* __restrict__ vc,
    const uint8_t* __restrict__ flags, const int32_t* __restrict__ Tpos,
    const int32_t* __restrict__ n_full, const int32_t* __restrict__ n_total, int n_qt, int B,
    int n_tokens, int Hq, int Hkv, int G, float bias_local, float bias_sink, bool xcd_order,
    float* __restrict__ part_o, float* __restrict__ part_ml, int2* __restrict__ seg_tab) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  using L = PPLds<D>;
  constexpr int KCH = D / 8;
  constexpr int ROWS = 1024 / (D * 2);
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;   // 0: group A, 1: group B
  const int P = B * G;

  // This workgroup's share of the work.  Segment (pair j, KV group g) has
  // len(j) = max(n_total) of the pair's query tiles; with up to 64 pairs
  // each lane holds one pair's length, prefix and n_full (one round of
  // loads at the start instead of a chain of dependent scalar loads).
  const int npairs = (n_qt + 1) / 2;
  auto pair_len = [&](int j) __attribute__((always_inline)) {
    const int a = n_total[2 * j];
    return 2 * j + 1 < n_qt ? max(a, n_total[2 * j + 1]) : a;
  };
  auto pair_nf = [&](int j) __attribute__((always_inline)) {
    const int a = n_full[2 * j];
    return 2 * j + 1 < n_qt ? min(a, n_full[2 * j + 1]) : a;
  };
  const bool lane_pairs = npairs <= 64;
  // Costs: a segment of len tiles costs len + kSkPieceCost units (its
  // piece's prologue and epilogue), the leading kSkPieceCost units being
  // virtual; workgroups split the units evenly.
  int len_l = 0, nf_l = 0, incl_l = 0;   // this lane's pair (lane < npairs); incl_l in units
  int lsum = 0;                          // units of one KV group's segments
  if (lane_pairs) {
    if (lane < npairs) {
      len_l = pair_len(lane);
      nf_l = pair_nf(lane);
    }
    incl_l = lane < npairs ? len_l + kSkPieceCost : 0;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl_l, o);
      if (lane >= o) incl_l += v;
    }
    lsum = __builtin_amdgcn_readlane(incl_l, 63);
  } else {
    for (int j = 0; j < npairs; ++j) lsum += pair_len(j) + kSkPieceCost;
  }
  auto seg_len = [&](int j) __attribute__((always_inline)) {
    return lane_pairs ? __builtin_amdgcn_readlane(len_l, j) : pair_len(j);
  };
  auto seg_nf = [&](int j) __attribute__((always_inline)) {
    return lane_pairs ? __builtin_amdgcn_readlane(nf_l, j) : pair_nf(j);
  };
  const long long T = static_cast<long long>(lsum) * Hkv;
  // At least kSkMinTiles units per workgroup, more than kSkPieceCost: every
  // range then holds a tile (the merge reads one piece from each workgroup
  // between the owners of a segment's first and last tile).
  static_assert(kSkMinTiles > kSkPieceCost, "ranges must reach past a segment's virtual units");
  const int W = static_cast<int>(
      max(1LL, min(static_cast<long long>(gridDim.x), T / kSkMinTiles)));
  const int w = xcd_order ? xcd_linear(blockIdx.x, gridDim.x) : static_cast<int>(blockIdx.x);
  if (w >= W) return;
  const long long r0 = w * T / W, r1 = (w + 1) * T / W;

  float m_eff = 0.f;
  bool m_set = false;
  bf16x8_t qx;
  auto set_qx = [&](float mref) __attribute__((always_inline)) {
    const bf16_t mh = f32_to_bf16(-mref);
    const bf16_t ml = f32_to_bf16(-mref - bf16_to_f32(mh));
    m_eff = -(bf16_to_f32(mh) + bf16_to_f32(ml));
    const bf16_t one = 0x3F80;
    const bf16_t v[8] = {one, one, mh, ml, 0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 8; ++i) qx[i] = __builtin_bit_cast(__bf16, half == 0 ? v[i] : static_cast<bf16_t>(0));
  };

  const size_t kv_row = static_cast<size_t>(Hkv) * D;
  const uint8_t* kg8 = nullptr;   // this piece's KV group
  const uint8_t* vg8 = nullptr;
  constexpr int KSL = kKvTile / ROWS;
  const size_t row_bytes = kv_row * 2;
  // DMA slices of this wave (waves 0-3 stage K, 4-7 stage V)
  auto slice_isv = [&](int j) __attribute__((always_inline)) { return wave * L::slices + j >= KSL; };
  uint32_t s_off[L::slices];
  int s_dst[L::slices];
#pragma unroll
  for (int j = 0; j < L::slices; ++j) {
    const int sl = wave * L::slices + j;
    const int row = (sl >= KSL ? sl - KSL : sl) * ROWS + lane / KCH, phys = lane % KCH;
    const int logical = slice_isv(j) ? vchunk<D>(row, phys) : kchunk<D>(row, phys);
    s_off[j] = static_cast<uint32_t>(row * row_bytes) + logical * 16;
    s_dst[j] = (slice_isv(j) ? L::vOff(0) : L::kOff(0)) + (sl >= KSL ? sl - KSL : sl) * 1024;
  }
  static_assert(L::kBytes == L::vBytes, "K and V stages advance by the same stride");
  constexpr int kRsrcWord3 = 0x00020000;
  // tile c into stage buf (as k_attn_mfma: wave 0 also brings the flag bytes)
  auto issue = [&](int c, int buf) __attribute__((always_inline)) {
    const int kv0 = c * kKvTile;
    const int rows = min(kKvTile, n_tokens - kv0);
    const int nbytes = rows * static_cast<int>(row_bytes);
    if (wave == 0) {
      if (rows == kKvTile) {
        if (lane < kKvTile / 4) {
          const __amdgpu_buffer_rsrc_t rf = __builtin_amdgcn_make_buffer_rsrc(
              const_cast<uint8_t*>(flags + kv0), 0, kKvTile, kRsrcWord3);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rf, KVR_LDS(lds + L::fOff(0) + buf * L::fBytes), 4, 4 * lane, 0,
                                                   0, 0);
        }
      } else {
        lds[L::fOff(0) + buf * L::fBytes + lane] = flags[min(kv0 + lane, n_tokens - 1)];
      }
    }
#pragma unroll
    for (int j = 0; j < L::slices; ++j) {
      const uint8_t* base = (slice_isv(j) ? vg8 : kg8) + static_cast<size_t>(kv0) * row_bytes;
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0, nbytes, kRsrcWord3);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, KVR_LDS(lds + buf * L::kBytes + s_dst[j]), 16,
                                               static_cast<int>(s_off[j]), 0, 0, 0);
    }
  };
  // this wave's part of the oldest tile in flight has landed; with `newer`,
  // the tile issued after it may still be in flight
  auto wait_tile = [&](bool newer) __attribute__((always_inline)) {
    if (newer) {
      if (wave == 0)
        attn_wait_vmcnt<L::slices + 1>();
      else
        attn_wait_vmcnt<L::slices>();
    } else {
      attn_wait_vmcnt<0>();
    }
  };

  uint32_t klane[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
    klane[ks] = lds_addr(lds) + L::kOff(0) + (lane & 31) * (D * 2) +
                (kchunk<D>(lane & 31, ks * 2 + half) << 4);
  const uint32_t flane = lds_addr(lds) + L::fOff(0) + (lane & 31);
  auto bias_word = [&](float b) __attribute__((always_inline)) {
    const bf16_t bh = f32_to_bf16(b);
    const bf16_t bl = f32_to_bf16(b - bf16_to_f32(bh));
    return half == 0 ? (static_cast<uint32_t>(bh) | (static_cast<uint32_t>(bl) << 16)) : 0u;
  };
  const uint32_t bw_l = bias_word(bias_local), bw_s = bias_word(bias_sink);
  const uint32_t bw_ls = bias_word(bias_local + bias_sink);
  const uint32_t bones = half == 0 ? 0x3F803F80u : 0u;
  auto bias_operand = [&](uint32_t f) __attribute__((always_inline)) {
    const uint32_t wl = (f & KVR_FLAG_SINK) ? bw_ls : bw_l;
    const uint32_t wn = (f & KVR_FLAG_SINK) ? bw_s : 0u;
    const uint32_t w = (f & KVR_FLAG_LOCAL) ? wl : wn;
    const u32x4_t v = {w, bones, 0u, 0u};
    return __builtin_bit_cast(bf16x8_t, v);
  };
  const int tr_key = (lane & 15) >> 2;
  const int tr_d = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  uint32_t vlane[D / 32];
  {
    const int key_l = 4 * half + tr_key;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int d = db * 32 + tr_d;
      vlane[db] = lds_addr(lds) + L::vOff(0) + key_l * (D * 2) + (vchunk<D>(key_l, d >> 3) << 4) +
                  (d & 7) * 2;
    }
  }

  bf16x8_t qf[D / 16];
  f32x16_t o[D / 32];
  float l = 0.f;
  f32x16_t s[2];          // scores of the tile between its product and softmax phases
  bf16x8_t pb[4];         // P of the tile between its softmax and PV phases
  int nf = 0, u = 0;

  // scores S^T = K Q^T + (bias - m_eff) of the tile in stage BUF
  auto qk = [&](auto bufc) __attribute__((always_inline)) {
    constexpr int BUF = decltype(bufc)::value;
    constexpr int KG = 4, GPS = D / 16 / KG, NG = 2 * GPS;
    uint32_t fb[2];
    fb[0] = ds_read_u8<BUF * L::fBytes>(flane);
    fb[1] = ds_read_u8<BUF * L::fBytes + 32>(flane);
    u32x4_t kb[2][KG];
    auto kread = [&](auto gic, u32x4_t(&dst)[KG]) {
      constexpr int gi = decltype(gic)::value, sb = gi / GPS, kq = gi % GPS;
      static_for<0, KG>([&](auto jc) __attribute__((always_inline)) {
        constexpr int j = decltype(jc)::value;
        dst[j] = ds_read_b128<L::kOff(BUF) + sb * 32 * D * 2>(klane[kq * KG + j]);
      });
    };
    kread(std::integral_constant<int, 0>{}, kb[0]);
    static_for<0, NG>([&](auto gic) __attribute__((always_inline)) {
      constexpr int gi = decltype(gic)::value, sb = gi / GPS, kq = gi % GPS;
      if constexpr (gi + 1 < NG) {
        kread(std::integral_constant<int, gi + 1>{}, kb[(gi + 1) & 1]);
        lds_wait_n<KG>();
      } else {
        lds_wait();
      }
#pragma unroll
      for (int j = 0; j < KG; ++j) reg_fence(kb[gi & 1][j]);
      if constexpr (gi == 0) {
        reg_fence(fb[0]);
        reg_fence(fb[1]);
      }
      if constexpr (kq == 0) {
#pragma unroll
        for (int t = 0; t < 16; ++t) s[sb][t] = 0.f;
      }
#pragma unroll
      for (int j = 0; j < KG; ++j)
        s[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kb[gi & 1][j]),
                                                         qf[kq * KG + j], s[sb], 0, 0, 0);
      if constexpr (kq == GPS - 1)
        s[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bias_operand(fb[sb]), qx, s[sb], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // O^T += V^T P^T for the tile in stage BUF
  auto pv = [&](auto bufc) __attribute__((always_inline)) {
    constexpr int BUF = decltype(bufc)::value;
    constexpr int NB = D / 32;
    u32x2_t xv[2][NB][2];
    auto vread = [&](auto stc, u32x2_t(&dst)[NB][2]) {
      constexpr int st = decltype(stc)::value, sb = st / 2, hs = st % 2;
      constexpr int off = BUF * L::vBytes + (sb * 32 + hs * 16) * D * 2;
      static_for<0, NB>([&](auto dbc) __attribute__((always_inline)) {
        constexpr int db = decltype(dbc)::value;
        dst[db][0] = ds_read_tr16<off>(vlane[db]);
        dst[db][1] = ds_read_tr16<off + 8 * D * 2>(vlane[db]);
      });
    };
    vread(std::integral_constant<int, 0>{}, xv[0]);
    static_for<0, 4>([&](auto stc) __attribute__((always_inline)) {
      constexpr int st = decltype(stc)::value;
      constexpr int NEXT = st + 1 < 4 ? 2 * NB : 0;
      auto& x = xv[st & 1];
      lds_wait_n<2 * (NB - 1)>();
      reg_fence(x[0][0]);
      reg_fence(x[0][1]);
      if constexpr (st + 1 < 4) vread(std::integral_constant<int, st + 1>{}, xv[(st + 1) & 1]);
      static_for<0, NB>([&](auto dbc) __attribute__((always_inline)) {
        constexpr int db = decltype(dbc)::value;
        if constexpr (db > 0) {
          lds_wait_n<2 * (NB - 1 - db) + NEXT>();
          reg_fence(x[db][0]);
          reg_fence(x[db][1]);
        }
        const u32x4_t w = {x[db][0][0], x[db][0][1], x[db][1][0], x[db][1][1]};
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, w), pb[st],
                                                         o[db], 0, 0, 0);
      });
    });
  };
  auto pv_at = [&](int buf) __attribute__((always_inline)) {
    static_for<0, kPPStages>([&](auto bc) __attribute__((always_inline)) {
      if (buf == decltype(bc)::value) pv(bc);
    });
  };

  // softmax of tile c: causal mask, lazy maximum, P and its row sum
  auto softmax = [&](int c) __attribute__((always_inline)) {
    if (c >= nf) {
      const int lim = u - c * kKvTile;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          const int kl = sb * 32 + 8 * (t >> 2) + 4 * half + (t & 3);
          if (kl > lim) s[sb][t] = -INFINITY;
        }
    }
    float mx[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      mx[i] = fmaxf(fmaxf(s[i >> 2][4 * (i & 3)], s[i >> 2][4 * (i & 3) + 1]),
                    fmaxf(s[i >> 2][4 * (i & 3) + 2], s[i >> 2][4 * (i & 3) + 3]));
    float mt = fmaxf(fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3])),
                     fmaxf(fmaxf(mx[4], mx[5]), fmaxf(mx[6], mx[7])));
    mt = xor32_max(mt);
    const bool bump = (mt > 8.f) || (!m_set && mt != -INFINITY);
    if (__builtin_amdgcn_ballot_w64(bump) != 0) {
      float shift = 0.f;
      if (bump) {
        const float old = m_eff;
        set_qx(m_eff + mt);
        shift = m_eff - old;
        const float corr = m_set ? fast_exp2(-shift) : 0.f;
        l *= corr;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int t = 0; t < 16; ++t) o[db][t] *= corr;
        m_set = true;
      }
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int t = 0; t < 16; ++t) s[sb][t] -= shift;
    }
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int t = 0; t < 16; ++t) s[sb][t] = fast_exp2(s[sb][t]);
    {
      float ps[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) ps[i] = s[i >> 3][2 * (i & 7)] + s[i >> 3][2 * (i & 7) + 1];
#pragma unroll
      for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
        for (int i = 0; i < w; ++i) ps[i] = ps[i] + ps[i + w];
      l += ps[0];
    }
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int i = 0; i < 8; ++i) pb[st][i] = static_cast<__bf16>(s[st / 2][(st % 2) * 8 + i]);
  };

  // Pieces: the parts of this workgroup's range that fall in one segment
  // (query-tile pair j, KV group g; segments in order g-major).
  int g = static_cast<int>(r0 / lsum), j = 0;
  long long start = static_cast<long long>(g) * lsum;
  int b0 = 0;   // stage of the piece's first tile: the ring continues across pieces
  if (lane_pairs) {
    // first pair whose inclusive prefix passes r0's offset in segment row g
    const unsigned long long past = __builtin_amdgcn_ballot_w64(lane < npairs && incl_l > r0 - start);
    j = __builtin_ctzll(past);
    start += __builtin_amdgcn_readlane(incl_l, j) - (__builtin_amdgcn_readlane(len_l, j) + kSkPieceCost);
  } else {
    while (start + pair_len(j) + kSkPieceCost <= r0) start += pair_len(j++) + kSkPieceCost;
  }
  for (;;) {
    // (the piece's scalars are wave-uniform; readfirstlane tells the compiler)
    j = __builtin_amdgcn_readfirstlane(j);
    g = __builtin_amdgcn_readfirstlane(g);
    const int len = __builtin_amdgcn_readfirstlane(seg_len(j));
    const long long tile0 = start + kSkPieceCost;   // unit of the segment's first tile
    const int c0 = __builtin_amdgcn_readfirstlane(static_cast<int>(max(r0, tile0) - tile0));
    const int n = __builtin_amdgcn_readfirstlane(static_cast<int>(min(r1, tile0 + len) - tile0) - c0);
    if (n <= 0) break;   // the range ends inside this segment's virtual units
    const int qt0 = 2 * j;
    // causal test from the first tile either query tile sees only partly
    nf = __builtin_amdgcn_readfirstlane(seg_nf(j));
    const int qt = qt0 + grp;
    kg8 = reinterpret_cast<const uint8_t*>(kc + static_cast<size_t>(g) * D);
    vg8 = reinterpret_cast<const uint8_t*>(vc + static_cast<size_t>(g) * D);
    // the query column this lane owns (past the last pair: a duplicate of
    // the last pair, computed and never written)
    const int p = qt * kQRows + (wave & 3) * 32 + (lane & 31);
    const int pc = min(p, P - 1);
    const int r = pc / G;
    const int h = g * G + (pc - r * G);
    // The query fragments and the position are loaded by instructions the
    // compiler does not track, ahead of the piece's first tile, and fenced
    // after that tile's wait (which they precede in issue order).  With
    // plain loads the compiler waited for them inside every tile's score
    // products (it cannot see that they completed in the first tile), and
    // its count there also held wave 0 on the flag bytes of the tile it
    // had just issued.
    uint32_t uraw = untracked_load_b32(Tpos + r);
    {
      const bf16_t* qrow = q + (static_cast<size_t>(r) * Hq + h) * D + 8 * half;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks)
        qf[ks] = __builtin_bit_cast(bf16x8_t, untracked_load_b128(qrow + ks * 16));
    }
    if (c0 == 0 && wave == 0 && lane == 0) {
      // the merge's view of this segment: its first workgroup and piece count
      const long long last = tile0 + len - 1;
      seg_tab[g * npairs + j] = make_int2(w, static_cast<int>(((last + 1) * W - 1) / T) - w + 1);
    }
    m_set = false;
    set_qx(0.f);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int t = 0; t < 16; ++t) o[db][t] = 0.f;
    l = 0.f;

    // Each wave runs the same program, tile by tile: a product phase (PV of
    // the previous tile, scores of this one) and a softmax phase, each ended by
    // a workgroup barrier.  Group B starts one barrier late (in phase 2i group
    // A takes the products of tile i while group B takes the softmax of tile
    // i - 1) and skips the barrier after its last softmax, so both pass 2n.
    // Each group issues its part of a tile at the start of a softmax phase:
    // group A tile i + 2 in phase 2i + 1, group B tile i + 3 in phase 2i + 2
    // (both into the stage that tile's predecessor by four left, whose last
    // reads ended a phase earlier), and at the end of phase 2i + 1 every wave
    // waits for its part of tile i + 1.
    issue(c0, b0);
    if (n > 1) issue(c0 + 1, (b0 + 1) % kPPStages);
    wait_tile(n > 1);
    reg_fence(uraw);
    u = static_cast<int>(uraw);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) reg_fence(qf[ks]);
    lds_barrier();
    if (grp == 1) {
      if (n > 2) issue(c0 + 2, (b0 + 2) % kPPStages);
      lds_barrier();
    }
    auto unit = [&](auto bc, int i) __attribute__((always_inline)) {
      constexpr int BUF = decltype(bc)::value;
      constexpr int PREV = (BUF + kPPStages - 1) % kPPStages;
      constexpr int NEXT2 = (BUF + 2) % kPPStages, NEXT3 = (BUF + 3) % kPPStages;
      // products (phase 2i for group A, 2i + 1 for group B), issued at a
      // raised wave priority so that the SIMD's arbiter prefers them to the
      // other wave's softmax
      __builtin_amdgcn_s_setprio(1);
      if (i > 0) pv(std::integral_constant<int, PREV>{});
      qk(bc);
      if (grp == 1 && i + 1 < n) wait_tile(i + 2 < n);
      lds_barrier();
      // softmax (phase 2i + 1 for group A, 2i + 2 for group B).  Both groups
      // issue their DMA here, so that the product phases carry no address
      // arithmetic (group A's tile i + 2 goes into the stage tile i - 2
      // left, whose last reads were B's PV in phase 2i - 1).
      __builtin_amdgcn_s_setprio(0);
      if (grp == 0 && i + 2 < n) issue(c0 + i + 2, NEXT2);
      if (grp == 1 && i + 3 < n) issue(c0 + i + 3, NEXT3);
      softmax(c0 + i);
      if (grp == 0 && i + 1 < n) wait_tile(i + 2 < n);
      if (grp == 0 || i + 1 < n) lds_barrier();
    };
    // tile i sits in stage (b0 + i) % kPPStages
    for (int k0 = 0; k0 < b0 + n; k0 += kPPStages) {
      static_for<0, kPPStages>([&](auto bc) __attribute__((always_inline)) {
        const int i = k0 + decltype(bc)::value - b0;
        if (i >= 0 && i < n) unit(bc, i);
      });
    }
    pv_at((b0 + n - 1) % kPPStages);   // PV of the last tile

    // partial of this piece: slot (segment + workgroup) * 2 + query tile of the pair
    const size_t slot = static_cast<size_t>(g * npairs + j + w) * 2 + grp;
    const int ql = (wave & 3) * 32 + (lane & 31);
    if (p < P) {
      // buffer stores: a lane offset plus a constant per element (no 64-bit
      // address per element, which the compiler would hoist and spill)
      const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
          part_o + slot * D * kQRows, 0, D * kQRows * 4, kRsrcWord3);
      const int vo = (4 * half * kQRows + ql) * 4;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          const float v = o[db][t];   // (bit_cast of a vector element reads element 0)
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), ro, vo,
                                                (db * 32 + 8 * (t >> 2) + (t & 3)) * kQRows * 4, 0);
        }
    }
    l = xor32_add(l);
    if (half == 0 && p < P) {
      float* pm = part_ml + slot * 2 * kQRows;
      pm[ql] = m_set ? m_eff : -INFINITY;
      pm[kQRows + ql] = l;
    }
    // No barrier here: the next piece's first three tiles go to the stages
    // after this piece's last one, which the other group may still be reading.
    b0 = (b0 + n) % kPPStages;
    start = tile0 + len;
    if (start >= r1) break;
    if (++j == npairs) {
      j = 0;
      ++g;
    }
  }
}

// Merge the split-KV partials: workgroup (query tile, KV group, kMergeD-row
// slice of d); thread (pair ql, 8 consecutive d).  Partial weights
// 2^(m_s - max m), normalised by the weighted sums; each thread writes its
// pair's 8 outputs (one 16-byte chunk of bf16, or two of float32).
constexpr int kMergeD = 8 * (kAttnThreads / kQRows);   // d rows per merge workgroup
static_assert(kAttnThreads % kQRows == 0, "merge threads cover whole query tiles");

template <int D, typename OutT>
__global__ __launch_bounds__(kAttnThreads) void k_attn_merge(
    const float* __restrict__ part_o, const float* __restrict__ part_ml,
    const int32_t* __restrict__ n_total, int n_qt, int B, int Hq, int Hkv, int G,
    int split_tiles, int n_splits, const int2* __restrict__ seg_tab, OutT* __restrict__ o) {
  const int qt = blockIdx.x, g = blockIdx.y;
  const int tid = threadIdx.x;
  const int ql = tid % kQRows;
  const int d0 = blockIdx.z * kMergeD + (tid / kQRows) * 8;
  const int p = qt * kQRows + ql;
  if (p >= B * G) return;
  // partials of this (query tile, KV group): slots slot0 + s * stride, s < ns
  int ns;
  size_t slot0, stride;
  if (seg_tab) {
    // stream-K pieces of segment s = (pair qt / 2, group g): one per workgroup
    // w0 .. w0 + ns - 1 (recorded by the attention kernel), in slot
    // (s + w) * 2 + qt % 2
    const int seg = g * ((n_qt + 1) / 2) + qt / 2;
    const int2 e = seg_tab[seg];
    ns = e.y;
    slot0 = static_cast<size_t>(seg + e.x) * 2 + (qt & 1);
    stride = 2;
  } else {
    ns = (n_total[qt] + split_tiles - 1) / split_tiles;
    slot0 = (static_cast<size_t>(qt) * Hkv + g) * n_splits;
    stride = 1;
  }
  // Partials four at a time with a running maximum (the sums so far are
  // rescaled when it grows): the four partials' maxima, sums and O values
  // are loaded together, indices past the last partial clamped to it and
  // their weights zeroed, so that a segment of up to four pieces (the usual
  // count) costs one round trip.  Partials that saw no key (maximum -inf)
  // add nothing.
  constexpr int kChunk = 4;
  float mmax = -INFINITY, denom = 0.f, acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  // (two chunks per iteration when there are more: the split kernel's
  // segments can have a dozen partials or more)
#pragma unroll 2
  for (int s0 = 0; s0 < ns; s0 += kChunk) {
    float ms[kChunk], ls[kChunk], ov[kChunk][8];
#pragma unroll
    for (int k = 0; k < kChunk; ++k) {
      const size_t sl = slot0 + static_cast<size_t>(min(s0 + k, ns - 1)) * stride;
      const float* pm = part_ml + sl * 2 * kQRows;
      const float* po = part_o + sl * D * kQRows + static_cast<size_t>(d0) * kQRows + ql;
      ms[k] = s0 + k < ns ? pm[ql] : -INFINITY;
      ls[k] = pm[kQRows + ql];
#pragma unroll
      for (int i = 0; i < 8; ++i) ov[k][i] = po[i * kQRows];
    }
    float mn = mmax;
#pragma unroll
    for (int k = 0; k < kChunk; ++k) mn = fmaxf(mn, ms[k]);
    const bool none = mn == -INFINITY;
    const float a = none ? 0.f : fast_exp2(mmax - mn);   // rescale of the sums so far
    denom *= a;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] *= a;
#pragma unroll
    for (int k = 0; k < kChunk; ++k) {
      const float w = none ? 0.f : fast_exp2(ms[k] - mn);   // 0 for ms = -inf
      denom += w * ls[k];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += w * ov[k][i];
    }
    mmax = mn;
  }
  const float inv = 1.f / denom;
  const int r = p / G, h = g * G + (p - r * G);
  OutT* dst = o + (static_cast<size_t>(r) * Hq + h) * D + d0;
  if constexpr (sizeof(OutT) == 2) {
    u32x4_t outv;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      outv[i] = static_cast<uint32_t>(f32_to_bf16(acc[2 * i] * inv)) |
                (static_cast<uint32_t>(f32_to_bf16(acc[2 * i + 1] * inv)) << 16);
    *reinterpret_cast<u32x4_t*>(dst) = outv;
  } else {
    reinterpret_cast<float4*>(dst)[0] = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
    reinterpret_cast<float4*>(dst)[1] = make_float4(acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
  }
}

// ---------------------------------------------------------------------------
// Inference-mode decode kernel: few pairs per KV head (B * G <= 64), the
// cache streamed once, HBM-bound.
//
// The keys 0..u_max a launch needs are cut into steps of 128; workgroup
// (c, g), one of W per KV head g, owns the steps [c * spw, (c + 1) * spw),
// and wave w of it takes the 32-key sub-tile w of each of its steps.  Every
// wave streams its own sub-tiles (K and V, 16 KB at d = 128, plus their
// flag bytes) through a ring of two LDS slots: the next sub-tile is in
// flight while the current one is used, so a CU keeps up to 128 KB on the
// way for as long as its range lasts (a long cache no longer takes several
// rounds of one-shot workgroups, each idling between its loads and the
// next workgroup's).  Queries are read in float32, scaled by
// log2(e)/sqrt(d) and rounded to bf16 once.  Per sub-tile a wave forms
// S^T = K Q^T for all pairs (one or two 32-pair column blocks), adds the
// log2(e)-scaled metadata bias, masks keys past each pair's position,
// updates its running (max, sum) and accumulates O^T = V^T P^T, with the
// operand layouts of the packed kernels (transposing reads for V^T).  LDS
// reads are inline assembly with explicit waits, so that the DMA into the
// other slot stays in flight.  At the end the four waves are combined
// through LDS and the workgroup writes one partial per pair;
// k_decode_merge combines the workgroups of each KV head.
// ---------------------------------------------------------------------------
constexpr int kDecSub = 32;                // keys per wave sub-tile
constexpr int kDecStep = 4 * kDecSub;      // keys per workgroup step
constexpr int kDecMaxPairs = 64;

template <int D>
struct DecLds {
  static constexpr int kBytes = kDecSub * D * 2;                     // K of one sub-tile
  static constexpr int slot = 2 * kBytes;                            // K then V
  static constexpr int wave = 2 * slot;                              // two slots per wave
  static constexpr int kv = 4 * wave;
  static constexpr int flags = 4 * 2 * kDecSub;                      // flag bytes per slot
  static constexpr int otRow = D + 4;                                // floats per pair row (padded)
  static constexpr int ot = 4 * kDecMaxPairs * otRow * 4;            // O of 4 waves
  static constexpr int body = kv + flags > ot ? kv + flags : ot;
  static constexpr int ml = 4 * kDecMaxPairs * 2 * 4;
  static constexpr int wt = kDecMaxPairs * 4 * 4;                    // per-pair wave weights
  static constexpr int total = body + ml + wt;
  static_assert(wave + slot < 65536, "ds offset field");
};

// Workgroups per KV head and steps per workgroup of a decode launch over
// n_tokens cached positions: one workgroup per CU in all, each with a
// contiguous run of steps.
struct DecGrid {
  int per_head, spw;
};
constexpr int kDecWorkgroups = 256;      // one per CU of an MI355X
DecGrid decode_grid(int n_tokens, const Shape& sh) {
  const int steps = (n_tokens + kDecStep - 1) / kDecStep;
  int per_head = kDecWorkgroups / sh.hkv;
  if (per_head < 1) per_head = 1;
  if (per_head > steps) per_head = steps;
  const int spw = (steps + per_head - 1) / per_head;
  return DecGrid{(steps + spw - 1) / spw, spw};
}

template <int D, int NCB>
__global__ __launch_bounds__(kAttnThreads, 1) void k_attn_decode(
    const float* __restrict__ q, const int32_t* __restrict__ pos, int B, int n_tokens,
    const bf16_t* __restrict__ kc, const bf16_t* __restrict__ vc,
    const uint8_t* __restrict__ flags, int Hq, int Hkv, int G, float q_scale, float bias_local,
    float bias_sink, int spw, float* __restrict__ part_o, float* __restrict__ part_ml) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  using L = DecLds<D>;
  constexpr int KCH = D / 8;                       // 16-byte chunks per row
  constexpr int ROWS = 1024 / (D * 2);             // rows per 1 KB DMA slice
  constexpr int KSL = kDecSub / ROWS;              // slices per operand per sub-tile
  constexpr int PAIRS = 32 * NCB;
  const int c = blockIdx.x, g = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int P = B * G;
  // this workgroup's steps [s0, s1max) of the cache (the grid has one per
  // workgroup, so s0 is a step of the cache); the ones past the last
  // query's position are dropped once the positions are in
  const int s0 = c * spw;
  const int s1max = min((n_tokens + kDecStep - 1) / kDecStep, s0 + spw);

  uint8_t* wbuf = lds + wave * L::wave;            // this wave's two slots
  uint8_t* fbuf = lds + L::kv + wave * 2 * kDecSub;
  float* ml = reinterpret_cast<float*>(lds + L::body);

  // queries of this lane's pair columns and their positions, loaded by
  // instructions the compiler does not track (its own wait for them would
  // drain the K/V loads issued after them); they are waited for explicitly,
  // behind the first sub-tiles, and their registers fenced before use
  u32x4_t qraw[NCB][D / 16][2];
  uint32_t uraw[NCB];
  uint32_t ulast = untracked_load_b32(pos + (B - 1));   // the last query's position
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const int p = min(cb * 32 + (lane & 31), P - 1);
    const int r = p / G;
    const int h = g * G + (p - r * G);
    uraw[cb] = untracked_load_b32(pos + r);
    const float* qrow = q + (static_cast<size_t>(r) * Hq + h) * D + 8 * half;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      qraw[cb][ks][0] = untracked_load_b128(qrow + ks * 16);
      qraw[cb][ks][1] = untracked_load_b128(qrow + ks * 16 + 4);
    }
  }

  // sub-tile j (keys j * kDecStep + wave * kDecSub ..) into slot b: its flag
  // bytes first (lanes 0..31), then K, then V.  Rows past the cache are
  // clamped to its last row (those keys are masked).
  const size_t kv_row = static_cast<size_t>(Hkv) * D;
  const bf16_t* kg = kc + static_cast<size_t>(g) * D;
  const bf16_t* vg = vc + static_cast<size_t>(g) * D;
  auto issue = [&](int j, int b) __attribute__((always_inline)) {
    const int key0 = j * kDecStep + wave * kDecSub;
    if (key0 + kDecSub <= n_tokens) {              // 32 flag bytes as 8 dwords
      if (lane < kDecSub / 4)
        __builtin_amdgcn_global_load_lds(KVR_GLB(flags + key0 + 4 * lane),
                                         KVR_LDS(fbuf + b * kDecSub), 4, 0, 0);
    } else if (lane < kDecSub) {                   // the cache's last sub-tile
      fbuf[b * kDecSub + lane] = flags[min(key0 + lane, n_tokens - 1)];
    }
#pragma unroll
    for (int sl = 0; sl < KSL; ++sl) {
      const int row = sl * ROWS + lane / KCH;
      const int key = min(key0 + row, n_tokens - 1);
      __builtin_amdgcn_global_load_lds(KVR_GLB(kg + key * kv_row + kchunk<D>(row, lane % KCH) * 8),
                                       KVR_LDS(wbuf + b * L::slot + sl * 1024), 16, 0, 0);
    }
#pragma unroll
    for (int sl = 0; sl < KSL; ++sl) {
      const int row = sl * ROWS + lane / KCH;
      const int key = min(key0 + row, n_tokens - 1);
      __builtin_amdgcn_global_load_lds(KVR_GLB(vg + key * kv_row + vchunk<D>(row, lane % KCH) * 8),
                                       KVR_LDS(wbuf + b * L::slot + L::kBytes + sl * 1024), 16, 0,
                                       0);
    }
  };
  constexpr int kIssued = 2 * KSL + 1;             // vector memory instructions per sub-tile

  // fragment addresses in slot 0 (slot 1 is an immediate offset away)
  uint32_t klane[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
    klane[ks] = lds_addr(wbuf) + (lane & 31) * (D * 2) + (kchunk<D>(lane & 31, ks * 2 + half) << 4);
  const int tr_key = (lane & 15) >> 2;
  const int tr_d = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  uint32_t vlane[2][2][D / 32];                    // [16-key half][8-key group][d block]
#pragma unroll
  for (int hs = 0; hs < 2; ++hs)
#pragma unroll
    for (int ins = 0; ins < 2; ++ins)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int key = hs * 16 + 8 * ins + 4 * half + tr_key;
        const int d = db * 32 + tr_d;
        vlane[hs][ins][db] = lds_addr(wbuf) + L::kBytes + key * (D * 2) +
                             (vchunk<D>(key, d >> 3) << 4) + (d & 7) * 2;
      }
  const uint32_t flane = lds_addr(fbuf) + (lane & 31);

  f32x16_t o[NCB][D / 32];
  float m[NCB], l[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    m[cb] = -INFINITY;
    l[cb] = 0.f;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int t = 0; t < 16; ++t) o[cb][db][t] = 0.f;
  }

  bf16x8_t qf[NCB][D / 16];                        // scaled queries (set below)
  int ucol[NCB];                                   // positions of the pair columns

  // one sub-tile from slot B; `next`: the following sub-tile is in flight
  // behind it (its K is waited for first, so the scores form while its V
  // lands)
  auto consume = [&](auto bc, int j, bool next) __attribute__((always_inline)) {
    constexpr int Bs = decltype(bc)::value;
    const int key0 = j * kDecStep + wave * kDecSub;
    if (next) attn_wait_vmcnt<KSL + kIssued>(); else attn_wait_vmcnt<KSL>();
    // K fragments and the flag byte of key lane & 31
    u32x4_t kf[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) kf[ks] = ds_read_b128<Bs * L::slot>(klane[ks]);
    uint32_t fl = ds_read_u8<Bs * kDecSub>(flane);
    lds_wait();
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) reg_fence(kf[ks]);
    reg_fence(fl);
    // bias of key kl (its flag byte was read by lane kl)
    const float bias_mine =
        ((fl & KVR_FLAG_LOCAL) ? bias_local : 0.f) + ((fl & KVR_FLAG_SINK) ? bias_sink : 0.f);
    float kbias[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) kbias[t] = __shfl(bias_mine, 8 * (t >> 2) + 4 * half + (t & 3), 64);
    f32x16_t sc[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
      for (int t = 0; t < 16; ++t) sc[cb][t] = 0.f;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks)
        sc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kf[ks]),
                                                         qf[cb][ks], sc[cb], 0, 0, 0);
      float mt = -INFINITY;
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const int kl = 8 * (t >> 2) + 4 * half + (t & 3);
        const float sv = sc[cb][t] + kbias[t];
        sc[cb][t] = (key0 + kl <= ucol[cb]) ? sv : -INFINITY;
        mt = fmaxf(mt, sc[cb][t]);
      }
      mt = xor32_max(mt);
      // Lazy running maximum: m moves only when the sub-tile exceeds it by
      // more than 8 (log2 units) or holds the column's first visible key,
      // so the weights stay below 2^8 and most sub-tiles leave O unscaled
      // (with two column blocks O lives in accumulation registers, where a
      // rescale reads, multiplies and writes back every element).  A column
      // that has seen no key yet keeps m = -inf and weight 0.
      const bool bump = mt > m[cb] + 8.f || (m[cb] == -INFINITY && mt != -INFINITY);
      if (__builtin_amdgcn_ballot_w64(bump) != 0) {
        const float mn = bump ? mt : m[cb];
        const float corr = m[cb] == -INFINITY ? 0.f : fast_exp2(m[cb] - mn);   // 1 if not bumped
        m[cb] = mn;
        l[cb] *= corr;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int t = 0; t < 16; ++t) o[cb][db][t] *= corr;
      }
      const bool none = m[cb] == -INFINITY;
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const float e = none ? 0.f : fast_exp2(sc[cb][t] - m[cb]);
        sc[cb][t] = e;
        l[cb] += e;
      }
    }
    // V^T fragments
    if (next) attn_wait_vmcnt<kIssued>(); else attn_wait_vmcnt<0>();
    u32x2_t vf[2][2][D / 32];
#pragma unroll
    for (int hs = 0; hs < 2; ++hs)
#pragma unroll
      for (int ins = 0; ins < 2; ++ins)
#pragma unroll
        for (int db = 0; db < D / 32; ++db) vf[hs][ins][db] = ds_read_tr16<Bs * L::slot>(vlane[hs][ins][db]);
    lds_wait();
#pragma unroll
    for (int hs = 0; hs < 2; ++hs)
#pragma unroll
      for (int ins = 0; ins < 2; ++ins)
#pragma unroll
        for (int db = 0; db < D / 32; ++db) reg_fence(vf[hs][ins][db]);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int hs = 0; hs < 2; ++hs) {
        bf16x8_t pb;
#pragma unroll
        for (int i = 0; i < 8; ++i) pb[i] = static_cast<__bf16>(sc[cb][hs * 8 + i]);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const u32x4_t w = {vf[hs][0][db][0], vf[hs][0][db][1], vf[hs][1][db][0], vf[hs][1][db][1]};
          o[cb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, w), pb,
                                                              o[cb][db], 0, 0, 0);
        }
      }
  };

  // the ring: sub-tile j in slot (j - s0) & 1; before a slot is refilled its
  // reads are complete (lds_wait in consume, then the compiler barrier).
  // The first two sub-tiles go out before the positions are known (they are
  // inside the cache whatever the positions say); s_hi bounds the sub-tiles
  // in flight, which can pass s1 when the last query sits early in the cache.
  issue(s0, 0);
  if (s0 + 1 < s1max) issue(s0 + 1, 1);
  const int s_hi = min(s0 + 2, s1max);
  // the queries and positions were issued before the sub-tiles in flight
  if (s_hi - s0 == 2) attn_wait_vmcnt<2 * kIssued>(); else attn_wait_vmcnt<kIssued>();
  reg_fence(ulast);
  const int nsteps = __builtin_amdgcn_readfirstlane(static_cast<int>(ulast)) / kDecStep + 1;
  if (s0 >= nsteps) {
    // every key here is in every pair's future: an empty partial (maximum
    // -inf, sum 0; the merge reads no O of it), and no DMA may land after
    // the exit
    const size_t slot0 = (static_cast<size_t>(c) * Hkv + g) * P;
    for (int p = tid; p < P; p += kAttnThreads) {
      part_ml[(slot0 + p) * 2] = -INFINITY;
      part_ml[(slot0 + p) * 2 + 1] = 0.f;
    }
    attn_wait_vmcnt<0>();
    return;
  }
  const int s1 = min(nsteps, s1max);               // steps holding a key 0..u_max
  const int s_end = max(s1, s_hi);
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    reg_fence(uraw[cb]);
    ucol[cb] = static_cast<int>(uraw[cb]);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      reg_fence(qraw[cb][ks][0]);
      reg_fence(qraw[cb][ks][1]);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        qf[cb][ks][i] = static_cast<__bf16>(__uint_as_float(qraw[cb][ks][i >> 2][i & 3]) * q_scale);
    }
  }
  for (int j = s0; j < s1; j += 2) {
    consume(std::integral_constant<int, 0>{}, j, j + 1 < s_end);
    asm volatile("" ::: "memory");
    if (j + 2 < s1) issue(j + 2, 0);
    if (j + 1 < s1) {
      consume(std::integral_constant<int, 1>{}, j + 1, j + 2 < s1);
      asm volatile("" ::: "memory");
      if (j + 3 < s1) issue(j + 3, 1);
    }
  }
  attn_wait_vmcnt<0>();
  __syncthreads();   // every wave is done with its slots: the LDS is reused below

  // per-wave (m, l) and O rows [pair][d] (row stride D + 4 floats; each lane
  // stores its accumulators' 4 consecutive d values as one 16-byte word)
  float* ot = reinterpret_cast<float*>(lds) + wave * kDecMaxPairs * L::otRow;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const int col = cb * 32 + (lane & 31);
    const float lt = xor32_add(l[cb]);             // both halves' keys
    if (half == 0) {
      ml[(wave * kDecMaxPairs + col) * 2] = m[cb];
      ml[(wave * kDecMaxPairs + col) * 2 + 1] = lt;
    }
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
        const int d = db * 32 + 8 * t4 + 4 * half;
        *reinterpret_cast<float4*>(ot + col * L::otRow + d) =
            make_float4(o[cb][db][4 * t4], o[cb][db][4 * t4 + 1], o[cb][db][4 * t4 + 2],
                        o[cb][db][4 * t4 + 3]);
      }
  }
  __syncthreads();

  const int npairs = min(P, PAIRS);
  const size_t slot0 = (static_cast<size_t>(c) * Hkv + g) * P;
  const float* ot_all = reinterpret_cast<const float*>(lds);
  // per pair: the four waves' weights exp2(m_w - M) (0 for a wave that saw
  // no key of it), stored for the O pass, and the partial's maximum and sum
  float* wt = ml + 4 * kDecMaxPairs * 2;
  for (int p = tid; p < npairs; p += kAttnThreads) {
    float mw[4], M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      mw[w] = ml[(w * kDecMaxPairs + p) * 2];
      M = fmaxf(M, mw[w]);
    }
    float e[4], ls = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      e[w] = mw[w] == -INFINITY ? 0.f : fast_exp2(mw[w] - M);
      ls += e[w] * ml[(w * kDecMaxPairs + p) * 2 + 1];
    }
    *reinterpret_cast<float4*>(wt + p * 4) = make_float4(e[0], e[1], e[2], e[3]);
    part_ml[(slot0 + p) * 2] = M;
    part_ml[(slot0 + p) * 2 + 1] = ls;
  }
  __syncthreads();
  // O: every load of an element's pass is independent of the others (one
  // LDS round trip per element instead of a chain through the maximum)
  for (int idx = tid; idx < npairs * (D / 4); idx += kAttnThreads) {
    const int p = idx / (D / 4), d = (idx - p * (D / 4)) * 4;
    const float4 e4 = *reinterpret_cast<const float4*>(wt + p * 4);
    const float e[4] = {e4.x, e4.y, e4.z, e4.w};
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float4 v = *reinterpret_cast<const float4*>(ot_all + (w * kDecMaxPairs + p) * L::otRow + d);
      acc.x += e[w] * v.x; acc.y += e[w] * v.y; acc.z += e[w] * v.z; acc.w += e[w] * v.w;
    }
    *reinterpret_cast<float4*>(part_o + (slot0 + p) * D + d) = acc;
  }
}

// Combines the workgroup partials of one (pair, KV head): every workgroup
// of the decode grid wrote one (those past the last query's position an
// empty one), so the count comes from the grid and no position is read.
// 1024 threads: thread (d, sg) takes the partials sg, sg + SG, ... (SG =
// 1024 / D groups), kChunk of them per round with their loads in flight
// together (index clamped, weight zeroed past the last) and a running
// maximum; the groups are then combined through LDS by group 0.
constexpr int kMergeThreads = 1024;

template <int D>
__global__ __launch_bounds__(kMergeThreads) void k_decode_merge(
    const float* __restrict__ part_o, const float* __restrict__ part_ml, int ns, int Hq, int Hkv,
    int G, int P, float* __restrict__ o) {
  constexpr int SG = kMergeThreads / D;
  constexpr int kChunk = 8;
  __shared__ float red_m[kMergeThreads];
  __shared__ float red_l[kMergeThreads];
  __shared__ float red_o[kMergeThreads];
  const int p = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
  const size_t stride = static_cast<size_t>(Hkv) * P;   // slots between workgroups
  const size_t slot0 = static_cast<size_t>(g) * P + p;
  const int d = tid % D, sg = tid / D;
  float m = -INFINITY, l = 0.f, acc = 0.f;
  for (int s = sg; s < ns; s += SG * kChunk) {
    float ms[kChunk], ls[kChunk], ov[kChunk];
#pragma unroll
    for (int k = 0; k < kChunk; ++k) {
      const size_t slot = slot0 + static_cast<size_t>(min(s + k * SG, ns - 1)) * stride;
      ms[k] = s + k * SG < ns ? part_ml[slot * 2] : -INFINITY;
      ls[k] = part_ml[slot * 2 + 1];
      ov[k] = part_o[slot * D + d];
    }
    float mn = m;
#pragma unroll
    for (int k = 0; k < kChunk; ++k) mn = fmaxf(mn, ms[k]);
    const bool none = mn == -INFINITY;
    const float a = none ? 0.f : fast_exp2(m - mn);    // rescale of the sums so far
    l *= a;
    acc *= a;
#pragma unroll
    for (int k = 0; k < kChunk; ++k) {
      // an empty partial adds nothing (its O is not read as a number)
      const bool empty = ms[k] == -INFINITY;
      const float b = empty ? 0.f : fast_exp2(ms[k] - mn);
      l += b * ls[k];
      acc += empty ? 0.f : b * ov[k];
    }
    m = mn;
  }
  red_m[tid] = m;
  red_l[tid] = l;
  red_o[tid] = acc;
  __syncthreads();
  if (sg == 0) {
    float M = -INFINITY;
#pragma unroll
    for (int j = 0; j < SG; ++j) M = fmaxf(M, red_m[tid + j * D]);
    float sum = 0.f, den = 0.f;
#pragma unroll
    for (int j = 0; j < SG; ++j) {
      const float mj = red_m[tid + j * D];
      const float e = mj == -INFINITY ? 0.f : fast_exp2(mj - M);
      den += e * red_l[tid + j * D];
      sum += e * red_o[tid + j * D];
    }
    const int r = p / G, h = g * G + (p - r * G);
    o[(static_cast<size_t>(r) * Hq + h) * D + d] = sum / den;
  }
}

// KV tiles per split: 32 (2048 keys) when the launch has plenty of
// workgroups; halved (down to 8) while the grid has fewer than 1024, so that
// small packed sets (few query tiles) still spread over every CU.  Roughly
// half of a causal grid exits at once (splits past a tile's last key).  Below
// 8 tiles a split's partial (66 KB per workgroup) costs more to write and
// merge than its share of the keys costs to attend.
int attn_split_tiles(int B, int n_tokens, const Shape& sh) {
  const long qk = static_cast<long>(plan_tiles(B, sh.group)) * sh.hkv;
  const int kv_tiles = (n_tokens + kKvTile - 1) / kKvTile;
  int st = 32;
  while (st > 8 && qk * ((kv_tiles + st - 1) / st) < 1024) st /= 2;
  return st;
}

// Workgroups of the stream-K pair kernel: one per CU, each taking an equal
// share of all (query-tile pair, KV group, KV tile) work; 0 for the split
// kernel.  The pair kernel is for d = 128 and launches with at least 16 KV
// tiles per CU at the cache's full length (below that the split kernel's
// 128-pair workgroups, two per CU, spread the work over more waves and a
// stream-K piece's prologue and epilogue weigh too much: 1.5B layer at 4K,
// 20.5 against 18.3 us).
int attn_sk_groups(int B, int n_tokens, const Shape& sh) {
  if (sh.d != 128) return 0;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  const long long tiles = static_cast<long long>(sh.hkv) * ((plan_tiles(B, sh.group) + 1) / 2) *
                          ((n_tokens + kKvTile - 1) / kKvTile);
  return tiles >= 16LL * cus ? cus : 0;
}

// Stream-K segments (query-tile pair, KV group); 0 for the split kernel.
size_t attn_segments(int B, int n_tokens, const Shape& sh) {
  return attn_sk_groups(B, n_tokens, sh) > 0
             ? static_cast<size_t>(sh.hkv) * ((plan_tiles(B, sh.group) + 1) / 2) : 0;
}

// Partial slots of one launch: stream-K pieces are numbered (segment +
// workgroup) per query tile of a pair; splits (query tile, KV group, split).
size_t attn_slots(int B, int n_tokens, const Shape& sh) {
  const int nt = plan_tiles(B, sh.group);
  const int W = attn_sk_groups(B, n_tokens, sh);
  if (W > 0) return static_cast<size_t>(sh.hkv * ((nt + 1) / 2) + W) * 2;
  const int st = attn_split_tiles(B, n_tokens, sh);
  const int ns = ((n_tokens + kKvTile - 1) / kKvTile + st - 1) / st;
  return static_cast<size_t>(nt) * sh.hkv * ns;
}

}  // namespace

bool decode_supported(kvr_dtype dt, int B, const Shape& sh) {
  return dt == KVR_BF16 && B >= 1 && static_cast<long>(B) * sh.group <= kDecMaxPairs;
}

size_t decode_workspace_bytes(int B, int n_tokens, const Shape& sh) {
  const size_t per_head = decode_grid(n_tokens, sh).per_head;
  return per_head * sh.hkv * B * sh.group * (sh.d + 2) * sizeof(float);
}

size_t attention_workspace_bytes(kvr_dtype dt, int B, int n_tokens, const Shape& sh) {
  if (dt != KVR_BF16) return 0;
  // partials (O, then max and sum), then the stream-K segment table
  return attn_slots(B, n_tokens, sh) * (sh.d + 2) * kQRows * sizeof(float) +
         attn_segments(B, n_tokens, sh) * sizeof(int2);
}

namespace {
template <int D>
hipError_t launch_mfma(const void* q, const void* k_cache, const void* v_cache,
                       const uint8_t* flags, const int32_t* T, int B, int n_tokens,
                       const Shape& sh, float alpha, float beta, const int32_t* n_full,
                       const int32_t* n_total, void* ws, hipStream_t stream) {
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_attn_mfma<D>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       AttnLds<D>::total);
    if (e != hipSuccess) return e;
    attr = true;
  }
  const int nt = plan_tiles(B, sh.group);
  const int st = attn_split_tiles(B, n_tokens, sh);
  const int ns = ((n_tokens + kKvTile - 1) / kKvTile + st - 1) / st;
  const size_t slots = attn_slots(B, n_tokens, sh);
  float* part_o = static_cast<float*>(ws);
  float* part_ml = part_o + slots * sh.d * kQRows;
  const float log2e = 1.4426950408889634f;
  if constexpr (D == 128) {
    const int sk = attn_sk_groups(B, n_tokens, sh);
    if (sk > 0) {
      static bool pp_attr = false;
      if (!pp_attr) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_attn_pp<D>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           PPLds<D>::total);
        if (e != hipSuccess) return e;
        pp_attr = true;
      }
      hipLaunchKernelGGL(k_attn_pp<D>, dim3(sk), dim3(kPPThreads), PPLds<D>::total,
                         stream, static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k_cache),
                         static_cast<const bf16_t*>(v_cache), flags, T, n_full, n_total, nt, B,
                         n_tokens, sh.hq, sh.hkv, sh.group, alpha * log2e, beta * log2e,
                         kAttnXcdOrder, part_o, part_ml,
                         reinterpret_cast<int2*>(part_ml + slots * 2 * kQRows));
      return hipGetLastError();
    }
  }
  dim3 grid(nt, sh.hkv, ns);
  hipLaunchKernelGGL(k_attn_mfma<D>, grid, dim3(kAttnMfmaThreads), AttnLds<D>::total, stream,
                     static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k_cache),
                     static_cast<const bf16_t*>(v_cache), flags, T, n_full, n_total, B, n_tokens,
                     sh.hq, sh.hkv, sh.group, alpha * log2e, beta * log2e, st, ns, part_o,
                     part_ml);
  return hipGetLastError();
}

template <int D, typename OutT>
hipError_t launch_merge(int B, int n_tokens, const Shape& sh, const int32_t* n_total, void* ws,
                        void* o_out, hipStream_t stream) {
  const int nt = plan_tiles(B, sh.group);
  const int st = attn_split_tiles(B, n_tokens, sh);
  const int ns = ((n_tokens + kKvTile - 1) / kKvTile + st - 1) / st;
  const size_t slots = attn_slots(B, n_tokens, sh);
  const float* part_o = static_cast<const float*>(ws);
  const float* part_ml = part_o + slots * sh.d * kQRows;
  hipLaunchKernelGGL((k_attn_merge<D, OutT>), dim3(nt, sh.hkv, D / kMergeD), dim3(kAttnThreads), 0,
                     stream, part_o, part_ml, n_total, nt, B, sh.hq, sh.hkv, sh.group, st, ns,
                     attn_sk_groups(B, n_tokens, sh) > 0
                         ? reinterpret_cast<const int2*>(part_ml + slots * 2 * kQRows)
                                            : nullptr,
                     static_cast<OutT*>(o_out));
  return hipGetLastError();
}
}  // namespace

namespace {
template <int D, int NCB>
hipError_t launch_decode_t(const float* q, const int32_t* pos, int B, int n_tokens,
                           const void* k_cache, const void* v_cache, const uint8_t* flags,
                           const Shape& sh, float alpha, float beta, void* ws, float* o,
                           hipStream_t stream) {
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_attn_decode<D, NCB>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       DecLds<D>::total);
    if (e != hipSuccess) return e;
    attr = true;
  }
  const DecGrid dg = decode_grid(n_tokens, sh);
  const int P = B * sh.group;
  float* part_o = static_cast<float*>(ws);
  float* part_ml = part_o + static_cast<size_t>(dg.per_head) * sh.hkv * P * sh.d;
  const float log2e = 1.4426950408889634f;
  hipLaunchKernelGGL((k_attn_decode<D, NCB>), dim3(dg.per_head, sh.hkv), dim3(kAttnThreads),
                     DecLds<D>::total, stream, q, pos, B, n_tokens,
                     static_cast<const bf16_t*>(k_cache), static_cast<const bf16_t*>(v_cache),
                     flags, sh.hq, sh.hkv, sh.group, log2e / sqrtf(static_cast<float>(D)),
                     alpha * log2e, beta * log2e, dg.spw, part_o, part_ml);
  return hipGetLastError();
}

template <int D>
hipError_t launch_decode_merge_t(int B, int n_tokens, const Shape& sh, void* ws, float* o,
                                 hipStream_t stream) {
  const DecGrid dg = decode_grid(n_tokens, sh);
  const int P = B * sh.group;
  const float* part_o = static_cast<const float*>(ws);
  const float* part_ml = part_o + static_cast<size_t>(dg.per_head) * sh.hkv * P * sh.d;
  hipLaunchKernelGGL(k_decode_merge<D>, dim3(P, sh.hkv), dim3(kMergeThreads), 0, stream, part_o,
                     part_ml, dg.per_head, sh.hq, sh.hkv, sh.group, P, o);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_attention_decode_merge(int B, int n_tokens, const Shape& sh, void* ws,
                                         float* o, hipStream_t stream) {
  if (sh.d == 128) return launch_decode_merge_t<128>(B, n_tokens, sh, ws, o, stream);
  return launch_decode_merge_t<64>(B, n_tokens, sh, ws, o, stream);
}

hipError_t launch_attention_decode(const float* q, const int32_t* pos, int B, int n_tokens,
                                   const void* k_cache, const void* v_cache,
                                   const uint8_t* flags, const Shape& sh, float alpha, float beta,
                                   void* ws, float* o, hipStream_t stream) {
  const bool two = B * sh.group > 32;
  if (sh.d == 128)
    return two ? launch_decode_t<128, 2>(q, pos, B, n_tokens, k_cache, v_cache, flags, sh, alpha,
                                         beta, ws, o, stream)
               : launch_decode_t<128, 1>(q, pos, B, n_tokens, k_cache, v_cache, flags, sh, alpha,
                                         beta, ws, o, stream);
  return two ? launch_decode_t<64, 2>(q, pos, B, n_tokens, k_cache, v_cache, flags, sh, alpha,
                                      beta, ws, o, stream)
             : launch_decode_t<64, 1>(q, pos, B, n_tokens, k_cache, v_cache, flags, sh, alpha,
                                      beta, ws, o, stream);
}

// Scale folded into Q by the RoPE kernel for the MFMA path.
float attention_q_scale(kvr_dtype dt, int head_dim) {
  return dt == KVR_BF16 ? 1.4426950408889634f / sqrtf(static_cast<float>(head_dim)) : 1.f;
}

hipError_t launch_attention(kvr_dtype dt, const void* q, const void* k_cache,
                            const void* v_cache, const uint8_t* flags, const int32_t* T, int B,
                            int n_tokens, const Shape& sh, float alpha, float beta,
                            const int32_t* plan_n_full, const int32_t* plan_n_total, void* ws,
                            void* o_out, hipStream_t stream) {
  if (B == 0) return hipSuccess;
  if (dt == KVR_BF16) {
    if (sh.d == 128)
      return launch_mfma<128>(q, k_cache, v_cache, flags, T, B, n_tokens, sh, alpha, beta,
                              plan_n_full, plan_n_total, ws, stream);
    return launch_mfma<64>(q, k_cache, v_cache, flags, T, B, n_tokens, sh, alpha, beta,
                           plan_n_full, plan_n_total, ws, stream);
  }
  hipLaunchKernelGGL(k_attn_rowwise<float>, dim3(B * sh.hq), dim3(64), 0, stream,
                     static_cast<const float*>(q), static_cast<const float*>(k_cache),
                     static_cast<const float*>(v_cache), flags, T, sh, alpha, beta,
                     static_cast<float*>(o_out));
  return hipGetLastError();
}

bool attention_needs_merge(kvr_dtype dt) { return dt == KVR_BF16; }

hipError_t launch_attention_merge(kvr_dtype dt, int B, int n_tokens, const Shape& sh,
                                  const int32_t* plan_n_total, void* ws, void* o_out,
                                  bool out_f32, hipStream_t stream) {
  if (B == 0 || dt != KVR_BF16) return hipSuccess;
  if (out_f32) {
    if (sh.d == 128) return launch_merge<128, float>(B, n_tokens, sh, plan_n_total, ws, o_out, stream);
    return launch_merge<64, float>(B, n_tokens, sh, plan_n_total, ws, o_out, stream);
  }
  if (sh.d == 128) return launch_merge<128, bf16_t>(B, n_tokens, sh, plan_n_total, ws, o_out, stream);
  return launch_merge<64, bf16_t>(B, n_tokens, sh, plan_n_total, ws, o_out, stream);
}

}  // namespace kvr
