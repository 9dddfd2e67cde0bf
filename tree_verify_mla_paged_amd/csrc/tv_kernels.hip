// Tree-masked verify attention over a paged MLA latent KV pool: gfx950 kernels.
//
// Computation (page 3 "The Pivot to Live Cutover", sections "The Technical
// Investigation" and "Input Knowledge Required"; page 2 "Flipping the Switch",
// section "The Long Road to Parity"): for every draft row (token t, head h) of
// request b, softmax over the visible gathered latent rows of sm_scale * q.k
// (576 dims), applied to the first 512 dims of those rows, plus the natural
// log-sum-exp.  Visibility is one mask byte per (draft, key), row stride L_b.
//
// Method: KV-split flash decoding with an LSE merge (page 2, section "The
// Broader Context").  Three kernels:
//   tv_pack_mask_kernel  mask bytes -> one 32-bit visibility word per
//                        (draft, 32-key tile), via wave ballots;
//   tv_split_kernel      one (request, 128-row block, KV split) per workgroup;
//   tv_merge_kernel      combines the splits of each row by their LSE.
//
// gfx950 mapping of tv_split_kernel
//  * 4 wave64s; wave w owns 32 query rows (rows of a request are (draft, head)
//    pairs, head fastest).  All 128 rows share each 32-key tile in LDS.
//  * Tiles are gathered by direct-to-LDS 16-byte loads (global_load_lds_dwordx4):
//    one instruction moves the 1024 bytes of a key's latent dims 0..511, one more
//    per wave moves the 64 RoPE dims of 8 keys, one moves the visibility words.
//    No registers hold in-flight tile data; three LDS stages (three distinct
//    __shared__ objects, the tile loop unrolled by three so every access names
//    its stage statically) keep two tiles in flight, and the compiler can see
//    that reads of one stage never wait for the gathers into another.
//  * S^T[key, row] = K[key, :] . Q[row, :] with v_mfma_f32_32x32x16_bf16:
//    A = key rows read from LDS (ds_read_b128), B = the wave's query rows held
//    in VGPRs for the whole split.  In the 32x32 accumulator layout lane l holds
//    row l % 32 and 16 of the 32 keys: the row max / sum is a 16-register
//    reduction plus one exchange with lane l ^ 32.
//  * O^T[d, row] += V^T[d, key] . P^T[key, row]: B = bf16 of those same 16
//    probabilities (no LDS round trip); A = V^T read straight from the
//    row-major tile with ds_read_b64_tr_b16 (within 16 lanes, output lane i
//    element j comes from source lane 4j + i/4, element i%4: when source lane
//    4j+q points at dims d0+4q.. of key j, lane i gets keys j=0..3 at dim d0+i).
//    O^T stays in the 256 accumulator registers (AGPRs) for the whole split.
//  * Reference maximum without rescaling: a row's reference is fixed at the
//    maximum of its first tile with a visible key (O and l are still exactly 0
//    then).  Probabilities exp2(x - ref) may grow to 2^TAU, which fp32 sums and
//    bf16 operands hold exactly in range, so O is never rescaled in the loop and
//    no VALU work ever touches the accumulators.  If some row's score exceeds
//    its reference by more than TAU, the workgroup restarts the split once with
//    each row's reference preset to its true maximum over the split (a QK-only
//    pass), after which probabilities are <= 1.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tv_kernels.h"

namespace tv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;

#define GLB_PTR(p) ((const __attribute__((address_space(1))) void*)(p))

constexpr int QK = 576;
constexpr int VD = 512;
constexpr int TILE = TILE_KEYS;
constexpr int ROW = 1280;                 // LDS bytes per key for latent dims 0..511
constexpr int MAIN_BYTES = TILE * ROW;    // 40960
constexpr int ROPE_BYTES = TILE * 128;    // RoPE dims 512..575 of 32 keys
constexpr int MASKW_BYTES = 4 * 64 * 4;   // 256 visibility words (one per draft)
constexpr int STAGE = MAIN_BYTES + ROPE_BYTES + MASKW_BYTES;  // 46080
constexpr int NSTAGE = 3;
constexpr int DMA_PER_TILE = 10;          // direct-to-LDS loads per wave per tile
constexpr float TAU = 64.0f;              // log2 headroom of a probability over its reference

// A key's 1024 latent bytes sit at key*ROW + key_shift(key).  With ROW a
// multiple of 256 bytes the shift alone picks the banks: the 16 keys of a QK
// read (same chunk) land on 16 distinct 16-byte bank groups, and the 4 keys of a
// transposed PV read (64 contiguous bytes each) on 4 distinct 64-byte groups.
// The shift is additive, so every read is a per-lane base plus an immediate.
__host__ __device__ constexpr int key_shift(int key) {
  return 64 * (key & 3) + 16 * ((key >> 2) & 3);
}
// XOR swizzle of the 8 RoPE chunks inside a key's 128-byte RoPE row.
__device__ __forceinline__ int rope_swz(int key) { return (key >> 1) & 7; }

// s_waitcnt vmcnt(n) leaving the other counters unconstrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 0xf) | ((N >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}

// ---------------------------------------------------------------- mask packing

// Word (token qo_indptr[b] + i, tile) bit k = mask byte of key 32*tile + k of draft i.
// Each half-wave (32 lanes) builds one word; keys at or past L_b give 0.
__global__ __launch_bounds__(256) void tv_pack_mask_kernel(PackParams p) {
  const int b = blockIdx.y;
  const int q0 = p.qo_indptr[b];
  const int n = p.qo_indptr[b + 1] - q0;
  const int L = p.kv_indptr[b + 1] - p.kv_indptr[b];
  const int tiles = (L + TILE - 1) / TILE;
  const int words = n * tiles;
  const int w = blockIdx.x * 8 + (threadIdx.x >> 5);
  const int k = threadIdx.x & 31;
  bool vis = false;
  int i = 0, tile = 0;
  if (w < words) {
    i = w / tiles;
    tile = w - i * tiles;
    const int key = tile * TILE + k;
    if (key < L) vis = p.mask[p.mask_indptr[b] + (int64_t)i * L + key] != 0;
  }
  const uint64_t bits = __ballot(vis);
  if (w < words && k == 0) {
    const uint32_t word = (threadIdx.x & 32) ? (uint32_t)(bits >> 32) : (uint32_t)bits;
    p.words[(int64_t)(q0 + i) * p.max_tiles + tile] = word;
  }
}

// ---------------------------------------------------------------- split kernel

// Everything a workgroup needs to gather and consume tiles of its KV split.
struct SplitCtx {
  const uint16_t* kv;
  const int32_t* idx;       // kv_indices of the request
  const uint32_t* wbase;    // visibility words of the block's first draft, split's first tile
  uint32_t wvoff;           // this lane's draft row offset (bytes) from wbase
  uint32_t voff;            // lane * 16: this lane's 16-byte chunk of a latent row
  int kbeg, kend, ntiles;   // key range [kbeg, kend) of the split, its 32-key tiles
  int wave, lane;
  // per-lane LDS offsets (relative to a stage)
  int qk_off, pv_off, mw_off, qr_off;
  int rp_off[4];
  bool row_ok;
  float scale_log2;
};

// Direct-to-LDS gathers, as inline asm: the compiler treats the equivalent
// builtin as an access that may complete out of order with LDS reads and then
// waits for all outstanding LDS reads (lgkmcnt(0)) wherever it needs any.
// Their completion is tracked explicitly with vmcnt instead (nothing else in
// the tile loop is a vector memory op).  M0 holds the LDS address; the global
// address is an SGPR base plus a 32-bit VGPR offset, or a 64-bit VGPR address.
template <int LDS_IMM>
__device__ __forceinline__ void dma16_s(uint32_t voff, const void* sbase, uint32_t m0base) {
  asm volatile("s_add_u32 m0, %2, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(m0base), "i"(LDS_IMM)
               : "m0");
}
__device__ __forceinline__ void dma16_v(const void* vaddr, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(vaddr), "s"(m0)
               : "m0");
}
__device__ __forceinline__ void dma4_s(uint32_t voff, const void* sbase, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(m0)
               : "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const lds_u8* p) { return (uint32_t)(uintptr_t)p; }

// Slots of this wave's 8 keys (8*wave .. 8*wave+7) of tile t: wave-uniform
// scalar loads, clamped to the split's last key.  Tiles past the split (the
// loop runs a multiple of 3 tiles) therefore gather real, finite rows, and their
// keys are masked off, so they contribute exactly 0.
__device__ __forceinline__ void load_slots(int (&slot)[8], const SplitCtx& c, int t) {
  const int kt = c.kbeg + t * TILE + 8 * c.wave;
#pragma unroll
  for (int i = 0; i < 8; ++i) slot[i] = c.idx[min(kt + i, c.kend - 1)];
}

// Latent dims 0..511 of key 8*wave + I go to stage + (8*wave + I)*ROW +
// key_shift(8*wave + I) = stage + [8*wave*ROW + 32*(wave & 1)] + LDS_IMM(I).
template <int I>
__device__ __forceinline__ void issue_main(const SplitCtx& c, const int (&slot)[8],
                                           uint32_t m0base) {
  constexpr int IMM = I * ROW + 64 * (I & 3) + 16 * (I >> 2);
  dma16_s<IMM>(c.voff, c.kv + (int64_t)slot[I] * QK, m0base);
  if constexpr (I + 1 < 8) issue_main<I + 1>(c, slot, m0base);
}

// Direct-to-LDS gather of tile t into stage sb: DMA_PER_TILE loads per wave.
// WIDE: the pool may exceed 4 GiB, so the RoPE gather (one slot per 8 lanes)
// uses 64-bit per-lane addresses; otherwise a 32-bit offset from the pool base.
template <bool WIDE>
__device__ __forceinline__ void issue_tile(lds_u8* sb, const int (&slot)[8], const SplitCtx& c,
                                           int t) {
  issue_main<0>(c, slot, lds_addr(sb) + 8 * c.wave * ROW + 32 * (c.wave & 1));
  {
    // recomputed every tile from an opaque copy of the lane id: a hoisted,
    // loop-invariant per-lane offset would be spilled, and its reload (a
    // vector memory op) would wait out the gathers just issued
    int lane = c.lane;
    asm volatile("" : "+v"(lane));
    const int j = lane >> 3;  // key 8*wave + j, RoPE chunk slot lane & 7
    int s = slot[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) s = (j == i) ? slot[i] : s;
    const int pos = 8 * c.wave + j;
    const uint32_t chunk = (uint32_t)((lane & 7) ^ rope_swz(pos));
    const uint32_t m0 = lds_addr(sb) + MAIN_BYTES + 8 * c.wave * 128;
    if constexpr (WIDE) {
      dma16_v(c.kv + (int64_t)s * QK + VD + chunk * 8, m0);
    } else {
      dma16_s<0>((uint32_t)s * (QK * 2) + VD * 2 + chunk * 16, c.kv, m0);
    }
  }
  dma4_s(c.wvoff, c.wbase + min(t, c.ntiles - 1),
         lds_addr(sb) + MAIN_BYTES + ROPE_BYTES + 256 * c.wave);
}

// The MFMAs of the tile loop are inline asm: S^T accumulates in VGPRs and O^T
// in the 256 AGPRs, which the compiler's own allocation does not achieve (it
// puts both in AGPRs and evicts an O block), and `volatile` keeps the LDS
// operand reads issued ahead of them where the source puts them.  Hazards the
// compiler cannot see are covered here: every MFMA starts with s_nop 1 (a
// VALU write of an operand register right before it); results are waited out
// (mfma_drain) before anything but another MFMA reads them.
__device__ __forceinline__ void mfma_acc_v(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_first_v(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_acc_a(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// >= 19 wait states: a 16-pass MFMA result may be read by VALU / v_accvgpr_read
__device__ __forceinline__ void mfma_drain_v(f32x16& acc) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(acc));
}

typedef const __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int QK_AHEAD = 4;  // (>= 4: the RoPE B operands are read inside the chain)
static_assert(true, "");  // LDS operand reads in flight ahead of the QK MFMA chain
constexpr int PV_AHEAD = 4;  // ... and ahead of the PV MFMAs

// Q's 64 RoPE dims live in LDS (QR_ROW bytes per query row, padded so the 16
// rows a QK read touches hit distinct banks); the 512 latent dims stay in VGPRs.
constexpr int QR_ROW = 144;

// S^T tile (32 keys x this wave's 32 rows) over all 576 dims.
__device__ __forceinline__ f32x16 qk_tile(const lds_u8* sb, const lds_u8* qrope,
                                          const bf16x8 (&qf)[VD / 16], const SplitCtx& c) {
  constexpr int NK = QK / 16;  // 36 k-steps: 32 latent (B in VGPRs), 4 RoPE (B in LDS)
  const lds_u8* qa = sb + c.qk_off;
  auto a_addr = [&](int ks) -> const lds_u8* {
    return ks < VD / 16 ? qa + 32 * ks : sb + c.rp_off[ks - VD / 16];
  };
  bf16x8 buf[QK_AHEAD], bq[4];
#pragma unroll
  for (int k = 0; k < QK_AHEAD; ++k) buf[k] = *reinterpret_cast<lds_bf16x8*>(a_addr(k));
  f32x16 acc;
#pragma unroll
  for (int ks = 0; ks < NK; ++ks) {
    const bf16x8 a = buf[ks % QK_AHEAD];
    const int nk = ks + QK_AHEAD;
    if (nk < NK) {
      buf[ks % QK_AHEAD] = *reinterpret_cast<lds_bf16x8*>(a_addr(nk));
      if (nk >= VD / 16)
        bq[nk - VD / 16] = *reinterpret_cast<lds_bf16x8*>(qrope + c.qr_off + 32 * (nk - VD / 16));
    }
    const bf16x8 b = ks < VD / 16 ? qf[ks] : bq[ks - VD / 16];
    if (ks == 0) mfma_first_v(acc, a, b);
    else mfma_acc_v(acc, a, b);
  }
  mfma_drain_v(acc);
  return acc;
}

// Visibility of the lane's row over tile t (bit k = key kbeg + 32*t + k).
__device__ __forceinline__ uint32_t tile_mask(const lds_u8* sb, const SplitCtx& c, int t) {
  const int rem = c.kend - (c.kbeg + t * TILE);
  const uint32_t valid = rem >= TILE ? 0xffffffffu : (rem <= 0 ? 0u : ((1u << rem) - 1u));
  const uint32_t w =
      *reinterpret_cast<const __attribute__((address_space(3))) uint32_t*>(sb + c.mw_off);
  return c.row_ok ? (w & valid) : 0u;
}

// Masked, scaled scores (log2 units) of the lane's 16 keys and their row max.
__device__ __forceinline__ float scores(float (&x)[16], const f32x16& acc, uint32_t mw,
                                        const SplitCtx& c) {
  const int half = c.lane >> 5;
  float tmax = -INFINITY;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int pos = 8 * (i >> 2) + 4 * half + (i & 3);  // accumulator row of register i
    x[i] = ((mw >> pos) & 1u) ? acc[i] * c.scale_log2 : -INFINITY;
    tmax = fmaxf(tmax, x[i]);
  }
  return fmaxf(tmax, __shfl_xor(tmax, 32));
}

// Pipeline head of tile t: once this wave's gathers of tile t have landed (at
// most tile t+1's are outstanding) and every wave has passed the barrier, the
// stage of tile t is readable and the stage of tile t-1 is free.
__device__ __forceinline__ void tile_head(const SplitCtx& c, int t, int nt) {
  if (t + 1 < nt) wait_vmcnt<DMA_PER_TILE>();
  else wait_vmcnt<0>();
  __syncthreads();
}

// Pipeline body of tile t in stage CUR: gather tile t+2 into stage (CUR+2)%3,
// then consume tile t.  m_true tracks each row's maximum over all tiles; a
// score above the row's reference by more than 2^TAU raises *flag (the pass is
// then redone with the reference preset to m_true; this pass's accumulators,
// possibly non-finite by then, are discarded).
template <int CUR, bool WIDE>
__device__ __forceinline__ void tile_body(lds_u8* const (&stages)[NSTAGE], int t, int nt,
                                          int (&slot)[8], const SplitCtx& c,
                                          const lds_u8* qrope, const bf16x8 (&qf)[VD / 16],
                                          f32x16 (&O)[VD / 32], float& m_ref, float& m_true,
                                          float& l_sum, int* flag) {
  if (t + 2 < nt) issue_tile<WIDE>(stages[(CUR + 2) % NSTAGE], slot, c, t + 2);
  const lds_u8* sb = stages[CUR];
  const uint32_t mw = tile_mask(sb, c, t);
  const f32x16 acc = qk_tile(sb, qrope, qf, c);
  float x[16];
  const float tmax = scores(x, acc, mw, c);
  m_true = fmaxf(m_true, tmax);
  if (m_ref == -INFINITY) m_ref = tmax;  // first visible keys: O and l are still 0
  if (__any(tmax > m_ref + TAU) && c.lane == 0) *flag = 1;
  const float mu = (m_ref == -INFINITY) ? 0.f : m_ref;
  bf16x8 pk[2];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float e = __builtin_amdgcn_exp2f(x[i] - mu);
    l_sum += e;
    pk[i >> 3][i & 7] = (__bf16)e;
  }
  // O^T += V^T . P^T; k-step kst covers keys 16*kst + {4*half + 0..3, 8 + 4*half + 0..3}.
  // MFMA m = 2*db + kst; its A operand is two transposed 8-byte reads.
  const lds_u8* va = sb + c.pv_off;
  auto pv_read = [&](int m) -> bf16x8 {
    const int db = m >> 1, kst = m & 1;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)(va + (16 * kst) * ROW + 64 * db));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)(va + (16 * kst + 8) * ROW + 32 + 64 * db));
    const bf16x4 l4 = __builtin_bit_cast(bf16x4, lo);
    const bf16x4 h4 = __builtin_bit_cast(bf16x4, hi);
    return bf16x8{l4[0], l4[1], l4[2], l4[3], h4[0], h4[1], h4[2], h4[3]};
  };
  constexpr int NM = VD / 16;  // 32 MFMAs
  bf16x8 vb[PV_AHEAD];
#pragma unroll
  for (int m = 0; m < PV_AHEAD; ++m) vb[m] = pv_read(m);
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    const bf16x8 a = vb[m % PV_AHEAD];
    if (m + PV_AHEAD < NM) vb[m % PV_AHEAD] = pv_read(m + PV_AHEAD);
    mfma_acc_a(O[m >> 1], a, pk[m & 1]);
  }
  // slots of tile t+3, for the gather issued by the next tile's body; loaded
  // last so no scalar load is outstanding while the LDS reads above pipeline
  if (t + 3 < nt) load_slots(slot, c, t + 3);
}

// All tiles of the split (c.ntiles >= 1), padded to a multiple of 3 with
// masked tiles; one exit, at the top (an exit between the tiles of a group
// costs the register allocator dearly).  Returns true if a restart is needed;
// every wave reads the flag after the same final barrier.
template <bool WIDE>
__device__ __forceinline__ bool run_split(lds_u8* const (&stages)[NSTAGE], const SplitCtx& c,
                                          const lds_u8* qrope, const bf16x8 (&qf)[VD / 16],
                                          f32x16 (&O)[VD / 32], float& m_ref, float& m_true,
                                          float& l_sum, int* flag) {
  const int nt = ((c.ntiles + NSTAGE - 1) / NSTAGE) * NSTAGE;
  int slot[8];
  load_slots(slot, c, 0);
  issue_tile<WIDE>(stages[0], slot, c, 0);
  load_slots(slot, c, 1);
  issue_tile<WIDE>(stages[1], slot, c, 1);
  load_slots(slot, c, 2);
  for (int t = 0; t < nt; t += NSTAGE) {
    tile_head(c, t, nt);
    tile_body<0, WIDE>(stages, t, nt, slot, c, qrope, qf, O, m_ref, m_true, l_sum, flag);
    tile_head(c, t + 1, nt);
    tile_body<1, WIDE>(stages, t + 1, nt, slot, c, qrope, qf, O, m_ref, m_true, l_sum, flag);
    tile_head(c, t + 2, nt);
    tile_body<2, WIDE>(stages, t + 2, nt, slot, c, qrope, qf, O, m_ref, m_true, l_sum, flag);
  }
  // drain: no gather may still be writing a stage when another pass reuses it
  wait_vmcnt<0>();
  __syncthreads();
  return *flag != 0;
}

template <int OUT, bool WIDE>
__global__ __launch_bounds__(256, 1) void tv_split_kernel(
    const uint16_t* __restrict__ q_, const uint16_t* __restrict__ kv_,
    const int32_t* __restrict__ kv_indices_, const int32_t* __restrict__ kv_indptr_,
    const int32_t* __restrict__ qo_indptr_, const uint32_t* __restrict__ mask_words_,
    void* __restrict__ out_, float* __restrict__ lse_, float* __restrict__ ws_o_,
    float* __restrict__ ws_lse_, SplitScalars p) {
  __shared__ __attribute__((aligned(1024))) uint8_t stage0[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t stage1[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t stage2[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t qrope_s[ROWS_PER_WG * QR_ROW];
  __shared__ int restart_flag;
  lds_u8* const stages[NSTAGE] = {(lds_u8*)stage0, (lds_u8*)stage1, (lds_u8*)stage2};
  lds_u8* const qrope = (lds_u8*)qrope_s;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int half = lane >> 5;

  // blockIdx -> work item: consecutive work items (the row blocks of one KV
  // split) go to the same XCD, which dispatch fills round-robin by blockIdx.
  const int per_xcd = gridDim.x / 8;
  const int work = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (work >= p.total_work) return;
  const int rb = work % p.row_blocks;
  const int s = (work / p.row_blocks) % p.max_splits;
  const int b = work / (p.row_blocks * p.max_splits);

  const int q0 = qo_indptr_[b];
  const int nq = qo_indptr_[b + 1] - q0;
  const int k0 = kv_indptr_[b];
  const int L = kv_indptr_[b + 1] - k0;
  const int H = p.num_heads;
  const int R = nq * H;
  const int row0 = rb * ROWS_PER_WG;
  if (row0 >= R) return;
  const int nsplit = L > 0 ? (L + p.split_keys - 1) / p.split_keys : 1;
  if (s >= nsplit) return;

  SplitCtx c;
  c.kv = kv_;
  c.idx = kv_indices_ + k0;
  c.kbeg = s * p.split_keys;
  c.kend = min(L, c.kbeg + p.split_keys);
  c.ntiles = c.kend > c.kbeg ? (c.kend - c.kbeg + TILE - 1) / TILE : 0;
  c.wave = wave;
  c.lane = lane;
  c.scale_log2 = p.scale_log2;

  const int i0 = row0 / H;
  const int nd = (min(row0 + ROWS_PER_WG, R) - 1) / H - i0 + 1;
  // this lane's query row
  const int r = row0 + wave * 32 + l32;
  c.row_ok = r < R;
  const int dl = c.row_ok ? r / H - i0 : 0;
  const int64_t g = (int64_t)q0 * H + r;  // global row = token * H + head
  // visibility words of draft i0 + d, tile 0 of the split: row (q0 + i0 + d)
  c.wbase = mask_words_ + (int64_t)(q0 + i0) * p.max_tiles + c.kbeg / TILE;
  c.wvoff = (uint32_t)min(64 * wave + lane, nd - 1) * (uint32_t)p.max_tiles * 4u;
  c.voff = (uint32_t)lane * 16u;

  // per-lane LDS read offsets (relative to a stage)
  c.qk_off = l32 * ROW + key_shift(l32) + 16 * half;  // + 32*ks: latent chunk 2*ks + half
#pragma unroll
  for (int j = 0; j < 4; ++j)  // RoPE chunk 2*j + half of key l32
    c.rp_off[j] = MAIN_BYTES + l32 * 128 + 16 * ((2 * j + half) ^ rope_swz(l32));
  // PV transposed reads: 16-lane group g16 = lane >> 4 picks dims +16*(g16 & 1);
  // source lane sl = lane & 15 points at key 4*half + sl/4, dims 4*(sl & 3)..+3.
  // Key 16*kst + 8*rd + 4*half + sl/4, dims 32*db + 16*(g16 & 1) + 4*(sl & 3):
  // pv_off + (16*kst + 8*rd)*ROW + 32*rd + 64*db  (key_shift is additive in rd)
  {
    const int sl = lane & 15;
    c.pv_off = (4 * half + (sl >> 2)) * ROW + 64 * (sl >> 2) + 16 * half +
               32 * ((lane >> 4) & 1) + 8 * (sl & 3);
  }
  c.mw_off = MAIN_BYTES + ROPE_BYTES + 4 * dl;

  // query rows -> MFMA B operands (k = dims 16*ks + 8*half .. +7): the 512
  // latent dims into VGPRs, the 64 RoPE dims of all 128 rows into LDS.  A row
  // past the request's rows uses the block's first row instead: its scores stay
  // in its own lane, are masked off, and it writes nothing.
  bf16x8 qf[VD / 16];
  {
    const int64_t gq = c.row_ok ? g : (int64_t)q0 * H + row0;
    const bf16x8* qp = reinterpret_cast<const bf16x8*>(q_ + gq * QK + half * 8);
#pragma unroll
    for (int ks = 0; ks < VD / 16; ++ks) qf[ks] = qp[2 * ks];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int id = tid + 256 * k;  // 128 rows x 8 RoPE chunks
      const int rl = id >> 3, ch = id & 7;
      const int64_t gr = (int64_t)q0 * H + (row0 + rl < R ? row0 + rl : row0);
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(q_ + gr * QK + VD + ch * 8);
      *reinterpret_cast<__attribute__((address_space(3))) bf16x8*>(qrope + rl * QR_ROW + ch * 16) = v;
    }
  }
  c.qr_off = (wave * 32 + l32) * QR_ROW + 16 * half;  // + 32*j: RoPE chunk 2*j + half
  __syncthreads();

  f32x16 O[VD / 32];
#pragma unroll
  for (int i = 0; i < VD / 32; ++i) O[i] = f32x16{};
  float m_ref = -INFINITY;  // reference maximum (log2 units)
  float l_sum = 0.f;        // this half's share of the normaliser
  if (c.ntiles > 0) {
    if (tid == 0) restart_flag = 0;
    __syncthreads();
    float m_pre = -INFINITY;
    for (int pass = 0; pass < 2; ++pass) {
      float m_true = -INFINITY;
      m_ref = m_pre;
      l_sum = 0.f;
#pragma unroll
      for (int i = 0; i < VD / 32; ++i) O[i] = f32x16{};
      if (!run_split<WIDE>(stages, c, qrope, qf, O, m_ref, m_true, l_sum, &restart_flag)) break;
      // a score exceeded its reference by more than 2^TAU: redo the split with
      // every row's reference at its true maximum (no score can exceed it)
      m_pre = m_true;
      if (tid == 0) restart_flag = 0;
      __syncthreads();
    }
  }

  // the last PV MFMAs must finish before O is read out of the AGPRs
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+a"(O[0]), "+a"(O[1]), "+a"(O[2]), "+a"(O[3]), "+a"(O[4]), "+a"(O[5]),
                 "+a"(O[6]), "+a"(O[7]), "+a"(O[8]), "+a"(O[9]), "+a"(O[10]), "+a"(O[11]),
                 "+a"(O[12]), "+a"(O[13]), "+a"(O[14]), "+a"(O[15]));
  const float l_tot = l_sum + __shfl_xor(l_sum, 32);
  const bool empty = !(l_tot > 0.f);
  const float inv = empty ? 0.f : 1.f / l_tot;
  // v_log_f32 is log2
  const float lse_nat = empty ? -INFINITY
                              : (m_ref + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994530942f;
  if (!c.row_ok) return;

  if (nsplit == 1) {
    if (half == 0) lse_[g] = lse_nat;
#pragma unroll
    for (int db = 0; db < VD / 32; ++db) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d0 = db * 32 + 8 * rq + 4 * half;
        f32x4 v;
        v[0] = O[db][4 * rq + 0] * inv;
        v[1] = O[db][4 * rq + 1] * inv;
        v[2] = O[db][4 * rq + 2] * inv;
        v[3] = O[db][4 * rq + 3] * inv;
        if (OUT == OUT_F32) {
          *reinterpret_cast<f32x4*>(static_cast<float*>(out_) + g * VD + d0) = v;
        } else {
          bf16x4 w;
          w[0] = (__bf16)v[0];
          w[1] = (__bf16)v[1];
          w[2] = (__bf16)v[2];
          w[3] = (__bf16)v[3];
          *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(out_) + g * VD + d0) = w;
        }
      }
    }
  } else {
    const int64_t ps = g * p.max_splits + s;
    if (half == 0) ws_lse_[ps] = lse_nat;
    float* po = ws_o_ + ps * VD;
#pragma unroll
    for (int db = 0; db < VD / 32; ++db) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d0 = db * 32 + 8 * rq + 4 * half;
        f32x4 v;
        v[0] = O[db][4 * rq + 0] * inv;
        v[1] = O[db][4 * rq + 1] * inv;
        v[2] = O[db][4 * rq + 2] * inv;
        v[3] = O[db][4 * rq + 3] * inv;
        *reinterpret_cast<f32x4*>(po + d0) = v;
      }
    }
  }
}

// ---------------------------------------------------------------- merge kernel

// One row per 128 threads; each thread owns 4 consecutive value dims and
// consumes the splits 8 at a time, so 8 independent loads are in flight.
template <int OUT>
__global__ __launch_bounds__(256) void tv_merge_kernel(MergeParams p) {
  constexpr int U = 8;
  const int b = blockIdx.y;
  const int q0 = p.qo_indptr[b];
  const int R = (p.qo_indptr[b + 1] - q0) * p.num_heads;
  const int r = blockIdx.x * 2 + (threadIdx.x >> 7);
  if (r >= R) return;
  const int L = p.kv_indptr[b + 1] - p.kv_indptr[b];
  const int ns = L > 0 ? (L + p.split_keys - 1) / p.split_keys : 1;
  if (ns <= 1) return;  // written directly by the split kernel
  const int64_t g = (int64_t)q0 * p.num_heads + r;
  const float* ls = p.ws_lse + g * p.max_splits;
  float M = -INFINITY;
  for (int s0 = 0; s0 < ns; s0 += U) {
    float v[U];
#pragma unroll
    for (int j = 0; j < U; ++j) v[j] = s0 + j < ns ? ls[s0 + j] : -INFINITY;
#pragma unroll
    for (int j = 0; j < U; ++j) M = fmaxf(M, v[j]);
  }
  const int d = (threadIdx.x & 127) * 4;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  float W = 0.f;
  if (M != -INFINITY) {
    const float* po = p.ws_o + g * p.max_splits * VD + d;
    for (int s0 = 0; s0 < ns; s0 += U) {
      float wgt[U];
      f32x4 v[U];
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const int s = s0 + j;
        // exp(-inf) = 0 for an empty split, whose partial output is not read
        wgt[j] = s < ns ? expf(ls[s] - M) : 0.f;
        v[j] = wgt[j] > 0.f ? *reinterpret_cast<const f32x4*>(po + (int64_t)s * VD)
                            : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int j = 0; j < U; ++j) {
        acc += wgt[j] * v[j];
        W += wgt[j];
      }
    }
    acc *= 1.f / W;
  }
  const float lse = (M == -INFINITY) ? -INFINITY : M + logf(W);
  if ((threadIdx.x & 127) == 0) p.lse[g] = lse;
  if (OUT == OUT_F32) {
    *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + g * VD + d) = acc;
  } else {
    bf16x4 w;
    w[0] = (__bf16)acc[0];
    w[1] = (__bf16)acc[1];
    w[2] = (__bf16)acc[2];
    w[3] = (__bf16)acc[3];
    *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(p.out) + g * VD + d) = w;
  }
}

// Launches go through hipLaunchKernel, which reports this launch's own status
// (a non-gfx950 device fails here: the library carries gfx950 code only).

hipError_t launch_pack(const PackParams& p, int grid_x, int batch, hipStream_t st) {
  PackParams a = p;
  void* args[] = {&a};
  return hipLaunchKernel(reinterpret_cast<const void*>(&tv_pack_mask_kernel), dim3(grid_x, batch),
                         dim3(256), args, 0, st);
}

hipError_t launch_split(const SplitParams& p, int grid, int out, hipStream_t st) {
  const uint16_t* q = p.q;
  const uint16_t* kv = p.kv;
  const int32_t* kvi = p.kv_indices;
  const int32_t* kvp = p.kv_indptr;
  const int32_t* qop = p.qo_indptr;
  const uint32_t* mw = p.mask_words;
  void* o = p.out;
  float* l = p.lse;
  float* wo = p.ws_o;
  float* wl = p.ws_lse;
  SplitScalars sc = p.s;
  void* args[] = {&q, &kv, &kvi, &kvp, &qop, &mw, &o, &l, &wo, &wl, &sc};
  const void* fn;
  if (p.wide)
    fn = out == OUT_F32 ? reinterpret_cast<const void*>(&tv_split_kernel<OUT_F32, true>)
                        : reinterpret_cast<const void*>(&tv_split_kernel<OUT_BF16, true>);
  else
    fn = out == OUT_F32 ? reinterpret_cast<const void*>(&tv_split_kernel<OUT_F32, false>)
                        : reinterpret_cast<const void*>(&tv_split_kernel<OUT_BF16, false>);
  return hipLaunchKernel(fn, dim3(grid), dim3(256), args, 0, st);
}

hipError_t launch_merge(const MergeParams& p, int grid_x, int batch, int out, hipStream_t st) {
  MergeParams a = p;
  void* args[] = {&a};
  const void* fn = out == OUT_F32 ? reinterpret_cast<const void*>(&tv_merge_kernel<OUT_F32>)
                                  : reinterpret_cast<const void*>(&tv_merge_kernel<OUT_BF16>);
  return hipLaunchKernel(fn, dim3(grid_x, batch), dim3(256), args, 0, st);
}

}  // namespace tv
