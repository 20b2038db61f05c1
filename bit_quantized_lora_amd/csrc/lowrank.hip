// ft_lowrank_fused: shared down-projection of the stabilizer and LoRA branches.
//
// FourTune section 3.3 ("LoRA Fusion"): the branches share their input, so one
// pass over it computes both down-projections:  out = [in wa^T | in wb^T]
// (forward: in = X, wa = L1^T, wb = A^T; backward: in = G, wa = L2, wb = B).
//
// HBM-bound (arithmetic intensity = rank FLOP/byte): the input is read exactly
// once.  A workgroup of 4 waves owns 64 rows and a contiguous range of
// 256-column chunks of the reduction: two row groups of 32, each split into two
// 128-column halves (column groups), so every row is fetched in 512-byte runs.
// (The dB variant, and ranks above 48, whose weight buffers and input staging
// would then crowd out the second workgroup per CU, keep 128 rows x 128
// columns: 4 row groups, one column group; see lowrank_plan.)  The split over the reduction gives the launch enough workgroups to
// keep every CU streaming.  Per chunk, the weight slices [rank x 128] are
// copied to LDS once (buffer_load ... lds, 16-byte-chunk XOR swizzle against
// bank conflicts) and shared by the waves, while each wave prefetches its own
// 32 x 128 input block of the next chunk into registers.  Products run on bf16
// MFMA 32x32x16 with fp32 accumulation; the column groups' partial products are
// added through LDS in column-group order.  Each split writes its partial sums
// to the workspace and a second pass adds the splits in a fixed order, so the
// result is deterministic.
//
// ft_quant_lowrank adds the 4-bit quantizer Q(in) (16x16 blocks, power-of-two
// scales, row-major E2M1 codes) to the same pass: a wave's 32 x 128 block is
// exactly 2 x 8 quantization blocks, already in registers for the
// down-projection, so the input is read from HBM once for both (the LoRA fusion
// of FourTune section 3.3 extended to the quantizer, which reads the same input).
// Lane (l32, lh) of a wave holds 8 values of its row group's row l32 in each 16-column
// block s; a block is spread over the 16 lanes of one DPP row and the matching
// 16 lanes of the other wave half, so its maximum is a 16-lane DPP reduction and
// one permlane32 swap across the halves.
//
// ft_quant_lowrank_db also takes the LoRA gradient dB = (X A)^T G (section 3.2)
// from the same registers in the backward's pass over G: the workgroup's
// 128 x 128 chunk of G goes to LDS row-major and comes back token-major through
// transposing reads (ds_read_b64_tr_b16), each wave multiplying (X A)^T of the
// workgroup's 128 tokens (from the forward's T, split into bf16 hi + lo like the
// GEMM epilogue's low-rank term) with 32 of the chunk's columns on bf16 MFMA.
// Each row block writes its partial dB for its columns; a second pass adds the
// row blocks in a fixed order.
//
// ft_gelu_quant_lowrank puts the activation between an MLP's two linears in
// front of that pass (FourTune section 3.3 "MLP Fusion": the intermediate is
// not read back by a separate kernel): the first linear's output Y is read,
// h = GELU(Y) is written out (the second linear's adapter gradient needs it)
// and quantized and projected from the same registers, so the 4608 x 12288
// intermediate crosses HBM once in each direction instead of three times.
#include "ft_device.h"

namespace ft {
namespace {

typedef __attribute__((address_space(3))) void lds_void;

constexpr int LR_THREADS = 256;
constexpr int LR_ROWS = 128;            // rows per workgroup (4 waves x 32)
constexpr int LR_CHUNK = 128;           // reduction columns per chunk (8 MFMA k-steps)
constexpr int LR_WROW = LR_CHUNK * 2;   // bytes per LDS weight row (256, swizzled, unpadded)
constexpr uint32_t RSRC_FLAGS = 0x00020000u;

#define FT_WAIT_VMCNT0() __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8))
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

__device__ __forceinline__ int wswz(int row, int q) { return row * LR_WROW + ((q ^ (row & 15)) << 4); }

// v_permlane32_swap exchanges the upper 32 lanes of its first operand with the
// lower 32 lanes of its second; with both operands v, lane l ends up with
// v[l mod 32] in the first result and v[32 + l mod 32] in the second.
__device__ __forceinline__ uint32_t other_half_max(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return max((uint32_t)r[0], (uint32_t)r[1]);
}
// the value of v in lane l ^ 32 (lh = l >> 5)
__device__ __forceinline__ uint32_t from_other_half(uint32_t v, int lh) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return lh ? (uint32_t)r[0] : (uint32_t)r[1];
}

typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;
typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));

// largest magnitude (as bf16 bits; magnitude order = integer order) of 8 bf16
// values: sign bits cleared, packed 16-bit maxima, then the two halves
__device__ __forceinline__ uint32_t abs_max8(const v4i& v) {
  const v2u16 a = __builtin_bit_cast(v2u16, (uint32_t)v.x & 0x7fff7fffu);
  const v2u16 b = __builtin_bit_cast(v2u16, (uint32_t)v.y & 0x7fff7fffu);
  const v2u16 c = __builtin_bit_cast(v2u16, (uint32_t)v.z & 0x7fff7fffu);
  const v2u16 d = __builtin_bit_cast(v2u16, (uint32_t)v.w & 0x7fff7fffu);
  const v2u16 m = __builtin_elementwise_max(__builtin_elementwise_max(a, b), __builtin_elementwise_max(c, d));
  return max((uint32_t)m.x, (uint32_t)m.y);
}

// wc: waves of a workgroup side by side along the reduction (1, 2 or 4): a
// workgroup owns LR_ROWS / wc rows and chunks of LR_CHUNK * wc columns
int64_t chunks_per_split(int64_t M, int64_t Kin, int wc = 1) {
  const int64_t nchunks = (Kin + LR_CHUNK * wc - 1) / (LR_CHUNK * wc);
  const int64_t rblocks = (M + LR_ROWS / wc - 1) / (LR_ROWS / wc);
  if (wc == 1) {
    int64_t s = (512 + rblocks - 1) / rblocks;        // aim for ~2 workgroups per CU
    if (s > nchunks) s = nchunks;
    if (s < 1) s = 1;
    int64_t cps = (nchunks + s - 1) / s;
    return cps < 4 ? (nchunks < 4 ? nchunks : 4) : cps;   // at least 4 chunks of work per split
  }
  // at most ~2 workgroups per CU, all resident at once
  int64_t s = 512 / rblocks;
  if (s > nchunks) s = nchunks;
  if (s < 1) s = 1;
  return (nchunks + s - 1) / s;
}

int64_t num_splits(int64_t M, int64_t Kin, int wc = 1) {
  const int64_t nchunks = (Kin + LR_CHUNK * wc - 1) / (LR_CHUNK * wc);
  const int64_t cps = chunks_per_split(M, Kin, wc);
  return (nchunks + cps - 1) / cps;
}

// the column-group width of the plain, quantizing and GELU passes (the dB
// variant keeps 128-row blocks): wide chunks give each row a longer contiguous
// run per request (512 bytes at wc 2), which the HBM serves faster than the
// 256-byte runs of 128-column chunks
constexpr int LR_WC = 2;

// dB partials of ft_quant_lowrank_db: the forward's T (fp32 [M x ldt], its LoRA
// columns from toff), the adapter rank r (1..64), partials [row blocks][r][Kin]
struct DbArgs {
  const float* T;
  int64_t ldt;
  int toff, r;
  float* part;
};

constexpr int DB_GPITCH = 2 * LR_CHUNK + 16;   // bytes per LDS row of the staged G chunk (conflict-free tr reads)

// NCT: 32-wide rank column tiles (0..4); QUANT: also write Q(in); GELU: the
// input is replaced by GELU(in) (written to hout [M x Kin]) before both; NDB:
// 32-row tiles of the dB partials (0: none; 1 for r <= 32, 2 for r <= 64);
// LINES: the input is loaded in whole 128-byte lines and re-laid out through
// LDS (below)
template <int NCT, bool QUANT, bool GELU = false, int NDB = 0, int WC = 1, bool LINES = false>
__global__ void __launch_bounds__(LR_THREADS)
lowrank_kernel(const uint16_t* __restrict__ in, int64_t M, int64_t Kin, int64_t ld_in,
               const uint16_t* __restrict__ wa, int ra, const uint16_t* __restrict__ wb, int rb,
               int64_t cps, float* __restrict__ out, int64_t out_split_stride,
               uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, uint16_t* __restrict__ hout,
               DbArgs db) {
  // WC waves side by side along the reduction: wave (rg, cq) = (wave / WC,
  // wave % WC) owns rows 32 rg .. of the workgroup's RB and columns
  // 128 cq .. of each CC-column chunk; its partial projection is added to the
  // other column groups' through LDS at the end, in cq order
  static_assert(WC == 1 || NDB == 0, "the dB variant uses 128-row blocks");
  static_assert(!LINES || NDB == 0, "the dB variant stages its G chunk itself");
  constexpr int RB = LR_ROWS / WC, CC = LR_CHUNK * WC;
  extern __shared__ __attribute__((aligned(1024))) uint8_t s_w[];   // 2 buffers of rho rows (+ dB staging)
  const int wslice = (ra + rb) * LR_WROW;          // one 128-column slice of the weight chunk
  const int wbuf_bytes = wslice * WC;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rg = wave / WC, cq = wave % WC;
  const int rho = ra + rb;
  const int l32 = lane & 31, lh = lane >> 5;
  const int64_t row0 = (int64_t)blockIdx.x * RB;
  const int64_t nchunks = (Kin + CC - 1) / CC;
  const int64_t c_begin = (int64_t)blockIdx.y * cps;
  const int64_t c_end = min(nchunks, c_begin + cps);

  const int64_t arow = row0 + 32 * rg + l32;
  const bool arow_ok = arow < M;
  // input rows of this workgroup through a buffer resource: a lane past M or past
  // the reduction gets an out-of-range offset and reads zeros (no branches)
  const __amdgpu_buffer_rsrc_t rIn = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(in + row0 * ld_in), 0, (int)(min<int64_t>(RB, M - row0) * ld_in * 2), RSRC_FLAGS);
  const uint32_t in_off = (uint32_t)(((32 * rg + l32) * ld_in + 8 * lh + 128 * cq) * 2);

  const __amdgpu_buffer_rsrc_t rWa =
      __builtin_amdgcn_make_buffer_rsrc((void*)wa, 0, (int)((int64_t)ra * Kin * 2), RSRC_FLAGS);
  const __amdgpu_buffer_rsrc_t rWb =
      __builtin_amdgcn_make_buffer_rsrc((void*)wb, 0, (int)((int64_t)rb * Kin * 2), RSRC_FLAGS);

  // weight chunk c -> LDS buffer, one [rho x 128-column] slice after the other:
  // DMA instruction i covers rank rows 4 (i / WC) .. +3 of slice i % WC; lane l
  // fills physical 16-byte chunk l & 15 of row 4 (i / WC) + l / 16
  auto issue_w = [&](int buf, int64_t c) {
    for (int i = wave; i < rho / 4 * WC; i += LR_THREADS / 64) {
      const int ri = i / WC, cs = i - ri * WC;
      const int row = 4 * ri + (lane >> 4);
      const int q = (lane & 15) ^ (row & 15);
      const int64_t col = c * CC + 128 * cs + 8 * q;
      const bool in_a = 4 * ri < ra;                  // ra is a multiple of 16: rows 4i..4i+3 share a matrix
      const int jj = in_a ? row : row - ra;
      const uint32_t off = col < Kin ? (uint32_t)(((int64_t)jj * Kin + col) * 2) : 0x80000000u;
      uint8_t* dst = s_w + buf * wbuf_bytes + cs * wslice + 4 * ri * LR_WROW;
      if (in_a) __builtin_amdgcn_raw_ptr_buffer_load_lds(rWa, (lds_void*)dst, 16, off, 0, 0, 0);
      else __builtin_amdgcn_raw_ptr_buffer_load_lds(rWb, (lds_void*)dst, 16, off, 0, 0, 0);
    }
  };
  // LINES: a wave's 32 x 128 block of a chunk is loaded in whole 128-byte lines
  // (instruction s covers rows 4 s + lr of the block, lr = lane / 16, 16 lanes x
  // 16 bytes per row); the fragment layout (32 rows x 32 bytes per instruction)
  // reads the same bytes at about half the rate.  relayout() then moves the
  // block through this wave's 8 KB of LDS staging into the MFMA fragment layout.
  const int lr = lane >> 4, lp = lane & 15;
  const uint32_t in_off_l = (uint32_t)(((32 * rg + lr) * ld_in + 8 * lp + 128 * cq) * 2);
  auto load_x = [&](v4i (&a)[8], int64_t c) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      if constexpr (LINES) {
        const int64_t k = c * CC + 128 * cq + 8 * lp;   // rows past M lie past the resource's range
        const uint32_t off = k < Kin ? in_off_l + (uint32_t)((4 * s * ld_in + c * CC) * 2) : 0x80000000u;
        a[s] = __builtin_amdgcn_raw_buffer_load_b128(rIn, off, 0, 2);   // nt: streamed, read once
      } else {
        const int64_t k = c * CC + 16 * s;              // + 128 cq (in in_off)
        const uint32_t off = (arow_ok && k + 128 * cq < Kin) ? in_off + (uint32_t)(k * 2) : 0x80000000u;
        a[s] = __builtin_amdgcn_raw_buffer_load_b128(rIn, off, 0, 0);
      }
    }
  };
  // whole-line layout -> fragment layout in place (lane (l32, lh) then holds row
  // l32, columns 16 s + 8 lh .. + 8 in x[s]): 256 bytes per staged row, its
  // 16-byte pieces XOR-swizzled by row so that the reads of 8 consecutive rows
  // fall in distinct banks.  Only this wave reads what it wrote; its LDS reads
  // are consumed before the next chunk's writes are issued.
  uint8_t* const stg = s_w + 2 * wbuf_bytes + wave * 8192;
  auto relayout = [&](v4i (&x)[8]) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int r = 4 * s + lr;
      *reinterpret_cast<v4i*>(stg + r * 256 + ((lp ^ (r & 7)) << 4)) = x[s];
    }
    compiler_fence();
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the block is in LDS
    compiler_fence();
#pragma unroll
    for (int s = 0; s < 8; ++s)
      x[s] = *reinterpret_cast<const v4i*>(stg + l32 * 256 + (((2 * s + lh) ^ (l32 & 7)) << 4));
  };

  // Codes and scales of a full chunk wait in registers and are stored after the
  // next chunk's barrier: the wait at the top of each chunk covers every
  // outstanding memory operation, so stores issued right before it would make
  // every chunk wait for a write round trip.
  struct Pending {
    v4i o0, o1;
    v2i s;
    uint8_t* codes;
    uint8_t* scales;
    bool live;
  } pend;
  pend.live = false;
  auto flush = [&]() {
    if (QUANT && pend.live) {
      *reinterpret_cast<v4i*>(pend.codes) = pend.o0;
      *reinterpret_cast<v4i*>(pend.codes + 16) = pend.o1;
      if (pend.scales) *reinterpret_cast<v2i*>(pend.scales) = pend.s;
      pend.live = false;
    }
  };

  // Q(in) of the chunk held in xa: one 16x16 block per (row half of the wave, s)
  auto quantize_chunk = [&](const v4i (&x)[8], int64_t c) {
    uint32_t cw[8];
    int ex[8];
    uint32_t mx[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      mx[s] = other_half_max(dpp_max16(abs_max8(x[s])));
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const uint32_t d[4] = {(uint32_t)x[s].x, (uint32_t)x[s].y, (uint32_t)x[s].z, (uint32_t)x[s].w};
      const int E = pow2_exp_bf16(mx[s]);
      ex[s] = E;
      const float sc = __builtin_bit_cast(float, (uint32_t)(E + 127) << 23);
      uint32_t w = 0;
      w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(w, __builtin_bit_cast(v2bf, d[0]), sc, 0);
      w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(w, __builtin_bit_cast(v2bf, d[1]), sc, 1);
      w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(w, __builtin_bit_cast(v2bf, d[2]), sc, 2);
      w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(w, __builtin_bit_cast(v2bf, d[3]), sc, 3);
      cw[s] = w;   // codes of columns 16s + 8lh .. +8 of this lane's row
    }
    if (!arow_ok) return;
    const int64_t k0 = c * CC + 128 * cq;
    uint8_t* crow = codes + arow * (Kin / 2) + k0 / 2;
    uint8_t* srow = scales + (arow / 16) * (Kin / 16) + k0 / 16;
    const bool sc_lane = lh == 0 && (l32 & 15) == 0;
    if (k0 + LR_CHUNK <= Kin) {
      // lane half 0 holds bytes [0, 32) of the row's 64 (blocks 0-3), half 1 bytes [32, 64);
      // the stores are issued after the next chunk's barrier (see pend)
      uint32_t r[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) r[k] = from_other_half(lh ? cw[k] : cw[k + 4], lh);
      if (lh == 0) {
        pend.o0 = v4i{(int)cw[0], (int)r[0], (int)cw[1], (int)r[1]};
        pend.o1 = v4i{(int)cw[2], (int)r[2], (int)cw[3], (int)r[3]};
      } else {
        pend.o0 = v4i{(int)r[0], (int)cw[4], (int)r[1], (int)cw[5]};
        pend.o1 = v4i{(int)r[2], (int)cw[6], (int)r[3], (int)cw[7]};
      }
      pend.s = v2i{(int)((ex[0] + 127) | (ex[1] + 127) << 8 | (ex[2] + 127) << 16 | (uint32_t)(ex[3] + 127) << 24),
                   (int)((ex[4] + 127) | (ex[5] + 127) << 8 | (ex[6] + 127) << 16 | (uint32_t)(ex[7] + 127) << 24)};
      pend.codes = crow + 32 * lh;
      pend.scales = sc_lane ? srow : nullptr;
      pend.live = true;
    } else {
#pragma unroll
      for (int s = 0; s < 8; ++s)
        if (k0 + 16 * s < Kin) *reinterpret_cast<uint32_t*>(crow + 8 * s + 4 * lh) = cw[s];
      if (sc_lane) {
#pragma unroll
        for (int s = 0; s < 8; ++s)
          if (k0 + 16 * s < Kin) srow[s] = (uint8_t)(ex[s] + 127);
      }
    }
  };

  // h = GELU(y) in place (fp32 math on the bf16 value, round to nearest even, as
  // ft_gelu_fwd), stored right away so the write overlaps the quantizer's and
  // the MFMAs' work
  auto gelu_chunk = [&](v4i (&x)[8], int64_t c) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const uint32_t w[4] = {(uint32_t)x[s].x, (uint32_t)x[s].y, (uint32_t)x[s].z, (uint32_t)x[s].w};
      uint32_t o[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        o[k] = f32_to_bf16_rne(gelu_f(bf16lo_to_f32(w[k]))) | (f32_to_bf16_rne(gelu_f(bf16hi_to_f32(w[k]))) << 16);
      x[s] = v4i{(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
      if constexpr (LINES) {   // whole-line layout: row 4 s + lr, 8 columns at 8 lp
        const int64_t row = row0 + 32 * rg + 4 * s + lr, k0 = c * CC + 128 * cq + 8 * lp;
        if (row < M && k0 < Kin) *reinterpret_cast<v4i*>(hout + row * Kin + k0) = x[s];
      } else {
        const int64_t k0 = c * CC + 128 * cq + 16 * s;
        if (arow_ok && k0 < Kin) *reinterpret_cast<v4i*>(hout + arow * Kin + k0 + 8 * lh) = x[s];
      }
    }
  };

  v16f acc[NCT > 0 ? NCT : 1];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) acc[ct] = v16f{};

  // dB: (X A)^T of this workgroup's 128 tokens as bf16 hi + lo planes [32 NDB][128]
  // in LDS after the weight buffers, then the G chunk [128][128] (pitch DB_GPITCH)
  uint8_t* s_t = s_w + 2 * wbuf_bytes;
  uint8_t* s_g = s_t + 2 * 32 * NDB * LR_ROWS * 2;
  if constexpr (NDB > 0) {
    for (int e = threadIdx.x; e < 32 * NDB * LR_ROWS; e += LR_THREADS) {
      const int j = e / LR_ROWS, m = e - j * LR_ROWS;
      const int64_t row = row0 + m;
      const float v = (j < db.r && row < M) ? db.T[row * db.ldt + db.toff + j] : 0.0f;
      uint32_t h, l;
      split_bf16(v, h, l);
      reinterpret_cast<uint16_t*>(s_t)[e] = (uint16_t)h;
      reinterpret_cast<uint16_t*>(s_t)[32 * NDB * LR_ROWS + e] = (uint16_t)l;
    }
  }

  // dB partial of chunk c: wave w takes the chunk's columns 32 w .. 32 w + 31 and
  // reduces over the workgroup's 128 tokens (8 k-steps of 16), A = (X A)^T hi and
  // lo from LDS, B = the G tile read token-major by transposing LDS reads; the
  // [r x 32] result goes to this row block's partial.  The tile was written by
  // all four waves, so a barrier comes first; the next chunk's barrier keeps it
  // intact until every wave has read it.
  auto dbp_chunk = [&](int64_t c) {
    if constexpr (NDB > 0) {
      // every wave's LDS writes of the tile visible; the next chunk's loads stay in flight
      compiler_fence();
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0), vmcnt and expcnt unconstrained
      __builtin_amdgcn_s_barrier();
      compiler_fence();
      const int g16 = lane >> 4, s16 = lane & 15;
      const int tr_row = 8 * (g16 >> 1) + (s16 >> 2);
      const int tr_col = 16 * (g16 & 1) + 4 * (s16 & 3);
      v16f dacc[NDB];
#pragma unroll
      for (int t = 0; t < NDB; ++t) dacc[t] = v16f{};
#pragma unroll
      for (int ks = 0; ks < LR_ROWS / 16; ++ks) {
        const uint8_t* b0 = s_g + (16 * ks + tr_row) * DB_GPITCH + 2 * (32 * wave + tr_col);
        const v4s lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(b0));
        const v4s hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(b0 + 4 * DB_GPITCH));
        const v2i l2 = __builtin_bit_cast(v2i, lo4), h2 = __builtin_bit_cast(v2i, hi4);
        const v8bf bq = __builtin_bit_cast(v8bf, v4i{l2.x, l2.y, h2.x, h2.y});
#pragma unroll
        for (int t = 0; t < NDB; ++t) {
          const int e = (32 * t + l32) * LR_ROWS + 16 * ks + 8 * lh;
          const v4i ah = *reinterpret_cast<const v4i*>(s_t + 2 * e);
          const v4i al = *reinterpret_cast<const v4i*>(s_t + 2 * (32 * NDB * LR_ROWS + e));
          dacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, ah), bq, dacc[t], 0, 0, 0);
          dacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, al), bq, dacc[t], 0, 0, 0);
        }
      }
      const int64_t col = c * LR_CHUNK + 32 * wave + l32;
      float* prow = db.part + (int64_t)blockIdx.x * db.r * Kin;
#pragma unroll
      for (int t = 0; t < NDB; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int j = 32 * t + 8 * (i >> 2) + 4 * lh + (i & 3);
          if (j < db.r && col < Kin) prow[(int64_t)j * Kin + col] = dacc[t][i];
        }
    }
  };

  // one chunk: wait for its DMA and loads, free the other buffer, start the next
  // chunk's loads into xn, then quantize and project xc (the two register sets
  // alternate, so nothing is copied between chunks)
  auto step = [&](v4i (&xc)[8], v4i (&xn)[8], int64_t c) {
    const int buf = (int)((c - c_begin) & 1);
    compiler_fence();
    FT_WAIT_VMCNT0();                    // this wave's DMA and loads of chunk c are done
    __builtin_amdgcn_s_barrier();        // every wave's DMA landed; buffer buf^1 is free
    compiler_fence();
    flush();
    if (c + 1 < c_end) {
      issue_w(buf ^ 1, c + 1);
      load_x(xn, c + 1);
    }
    if constexpr (GELU) gelu_chunk(xc, c);
    if constexpr (NDB > 0) {   // this wave's 32 rows of the chunk into the LDS tile, row-major
#pragma unroll
      for (int s = 0; s < 8; ++s)
        *reinterpret_cast<v4i*>(s_g + (32 * wave + l32) * DB_GPITCH + (16 * s + 8 * lh) * 2) = xc[s];
    }
    if constexpr (LINES) relayout(xc);
    if constexpr (QUANT) quantize_chunk(xc, c);
    const uint8_t* wbuf = s_w + buf * wbuf_bytes + cq * wslice;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const int j = 32 * ct + l32;
        const v4i b = j < rho ? *reinterpret_cast<const v4i*>(wbuf + wswz(j, 2 * s + lh)) : v4i{0, 0, 0, 0};
        acc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, xc[s]),
                                                          __builtin_bit_cast(v8bf, b), acc[ct], 0, 0, 0);
      }
    }
    if constexpr (NDB > 0) dbp_chunk(c);
  };
  v4i xa[8], xb[8];
  if (c_begin < c_end) {
    issue_w(0, c_begin);
    load_x(xa, c_begin);
  }
  for (int64_t c = c_begin; c < c_end; c += 2) {
    step(xa, xb, c);
    if (c + 1 < c_end) step(xb, xa, c + 1);
  }

  flush();
  if constexpr (WC > 1 && NCT > 0) {
    // the column groups' partial projections, added in cq order by the cq = 0 wave
    compiler_fence();
    __syncthreads();                                  // every wave done with the weight buffers
    float* red = reinterpret_cast<float*>(s_w);       // [wave][NCT][16][64]
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int r = 0; r < 16; ++r) red[((wave * NCT + ct) * 16 + r) * 64 + lane] = acc[ct][r];
    __syncthreads();
    if (cq == 0) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float v = acc[ct][r];
#pragma unroll
          for (int q = 1; q < WC; ++q) v += red[(((wave + q) * NCT + ct) * 16 + r) * 64 + lane];
          acc[ct][r] = v;
        }
    }
  }
  float* o = out + (int64_t)blockIdx.y * out_split_stride;
  if (WC > 1 && cq != 0) return;
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const int j = 32 * ct + l32;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t row = row0 + 32 * rg + 8 * (r >> 2) + 4 * lh + (r & 3);
      if (row < M && j < rho) o[row * rho + j] = acc[ct][r];
    }
  }
}

// out = sum over the splits of part[s], added in split order 0, 1, ... from 0.0f
// (deterministic).  n is a multiple of 4 (M and the rank are multiples of 16):
// each thread adds 4 consecutive values with 16-byte loads, the split loop
// unrolled so that its loads are in flight together.
__global__ void sum_splits_kernel(const float* __restrict__ part, int64_t splits, int64_t n, float* __restrict__ out) {
  const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i >= n) return;
  v4f v = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 8
  for (int64_t s = 0; s < splits; ++s) v += *reinterpret_cast<const v4f*>(part + s * n + i);
  *reinterpret_cast<v4f*>(out + i) = v;
}

}  // namespace
}  // namespace ft

// split partials of either block shape (128-row blocks for the dB variant and
// above 48 ranks, LR_WC column groups otherwise)
extern "C" size_t ft_lowrank_workspace(int64_t M, int64_t Kin, int32_t rho) {
  using namespace ft;
  if (M <= 0 || Kin <= 0 || rho <= 0) return 0;
  int64_t S = num_splits(M, Kin, 1);
  const int64_t S2 = num_splits(M, Kin, LR_WC);
  if (S2 > S) S = S2;
  return S > 1 ? (size_t)(S * M * rho * sizeof(float)) : 0;
}

namespace ft {
namespace {
int64_t row_blocks(int64_t M) { return (M + LR_ROWS - 1) / LR_ROWS; }

// The launch layout of a pass over in [M x Kin] projecting onto rho ranks (db: the
// dB-fold variant).  Column groups double the weight buffers, and whole-line
// loads add 32 KB of input staging: both are taken where two workgroups still
// fit a CU (column groups with whole-line loads up to rank 48, 128-row blocks
// with them up to rank 96); higher ranks and the dB variant keep 128-row blocks
// and the fragment-layout loads.  LDS: two weight chunks of wc slices, the
// staging after them, and for wc > 1 the column groups' partial projections,
// which reuse the space after the last chunk.
struct LrPlan {
  int wc = 1;
  bool lines = false;
  int64_t cps = 0, splits = 0;
  size_t lds = 0;
};
constexpr size_t kLdsPerWg = 80 * 1024, kStage = (size_t)(LR_THREADS / 64) * 8192;

LrPlan lowrank_plan(int64_t M, int64_t Kin, int rho, bool db) {
  LrPlan pl;
  const auto w_bytes = [&](int w) { return (size_t)2 * rho * LR_WROW * w; };
  if (!db) {
    if (w_bytes(LR_WC) + kStage <= kLdsPerWg) { pl.wc = LR_WC; pl.lines = true; }
    else if (w_bytes(1) + kStage <= kLdsPerWg) { pl.wc = 1; pl.lines = true; }
  }
  pl.cps = chunks_per_split(M, Kin, pl.wc);
  pl.splits = num_splits(M, Kin, pl.wc);
  const size_t lds_w = w_bytes(pl.wc) + (pl.lines ? kStage : 0);
  const size_t lds_red =
      pl.wc > 1 ? (size_t)(LR_THREADS / 64) * ((rho + 31) / 32) * 16 * 64 * sizeof(float) : 0;
  pl.lds = lds_w > lds_red ? lds_w : lds_red;
  return pl;
}

ft_status lowrank_impl(const void* in, int64_t M, int64_t Kin, int64_t ld_in, const void* wa, int32_t ra,
                       const void* wb, int32_t rb, float* out, uint8_t* codes, uint8_t* scales, void* workspace,
                       size_t ws_bytes, hipStream_t stream, void* hout = nullptr, const DbArgs* dbp = nullptr,
                       float* dB = nullptr) {
  if (!mult16(M) || !mult16(Kin) || ld_in < Kin) return FT_ESHAPE;
  if (ra < 0 || rb < 0 || (ra % 16) || (rb % 16) || ra + rb > 128) return FT_ESHAPE;
  const int rho = ra + rb;
  const bool quant = codes != nullptr;
  if (M == 0 || (rho == 0 && !quant)) return FT_OK;
  if ((rho && !out) || (ra && !wa) || (rb && !wb) || (Kin && !in) || (quant && !scales)) return FT_EINVAL;
  if ((Kin && !aligned16(in)) || (ld_in % 8) || (ra && !aligned16(wa)) || (rb && !aligned16(wb)) ||
      (rho && !aligned16(out)) || (quant && (!aligned16(codes) || !aligned16(scales))))
    return FT_EALIGN;
  if (hout && !aligned16(hout)) return FT_EALIGN;
  if (Kin == 0) return rho ? fill_zero_f32(out, M * rho, stream) : FT_OK;  // empty reduction
  if ((int64_t)rho * Kin * 2 >= ((int64_t)1 << 31)) return FT_ESHAPE;
  const size_t need_v = rho ? ft_lowrank_workspace(M, Kin, rho) : 0;
  const size_t off_db = (need_v + 255) & ~(size_t)255;
  const size_t need = dbp ? off_db + (size_t)row_blocks(M) * dbp->r * Kin * sizeof(float) : need_v;
  if (need && (!workspace || ws_bytes < need)) return workspace ? FT_ESPACE : FT_EINVAL;
  if (need && !aligned16(workspace)) return FT_EALIGN;
  DbArgs db{};
  if (dbp) {
    db = *dbp;
    db.part = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + off_db);
  }
  const LrPlan pl = lowrank_plan(M, Kin, rho, dbp != nullptr);
  const int wc = pl.wc;
  const bool lines = pl.lines;
  const int64_t cps = pl.cps;
  const int64_t S = pl.splits;
  float* dst = (S > 1 && rho) ? static_cast<float*>(workspace) : out;
  dim3 grid((unsigned)((M + LR_ROWS / wc - 1) / (LR_ROWS / wc)), (unsigned)S);
  const size_t lds_wc = pl.lds;
  const uint16_t* ip = static_cast<const uint16_t*>(in);
  const uint16_t* a = static_cast<const uint16_t*>(wa);
  const uint16_t* b = static_cast<const uint16_t*>(wb);
  const int64_t stride = M * rho;
  const int nct = (rho + 31) / 32;
  uint16_t* hp = static_cast<uint16_t*>(hout);
#define FT_LR_ONE(N, Q, G, W, L)                                                                             \
  hipLaunchKernelGGL((lowrank_kernel<N, Q, G, 0, W, L>), grid, dim3(LR_THREADS), lds_wc, stream, ip, M, Kin, ld_in, \
                     a, ra, b, rb, cps, dst, stride, codes, scales, hp, db)
#define FT_LR_ANY(N, Q, G)                          \
  if (wc > 1 && lines) { FT_LR_ONE(N, Q, G, LR_WC, true); }  \
  else if (lines) { FT_LR_ONE(N, Q, G, 1, true); }  \
  else { FT_LR_ONE(N, Q, G, 1, false); }
#define FT_LR_LAUNCH(N, Q) FT_LR_ANY(N, Q, false)
#define FT_LRG_LAUNCH(N) FT_LR_ANY(N, true, true)
  // dB partials: + (X A)^T hi/lo planes and the staged G chunk
#define FT_LRD_LAUNCH(N, D)                                                                                  \
  hipLaunchKernelGGL((lowrank_kernel<N, true, false, D>), grid, dim3(LR_THREADS),                          \
                     (size_t)(2 * rho * LR_WROW + 2 * 32 * D * LR_ROWS * 2 + LR_ROWS * DB_GPITCH), stream, ip, M, Kin, \
                     ld_in, a, ra, b, rb, cps, dst, stride, codes, scales, hp, db)
  if (dbp) {
    const int ndb = (db.r + 31) / 32;
#define FT_LRD_SWITCH(D)                        \
    switch (nct) {                              \
      case 0: FT_LRD_LAUNCH(0, D); break;       \
      case 1: FT_LRD_LAUNCH(1, D); break;       \
      case 2: FT_LRD_LAUNCH(2, D); break;       \
      case 3: FT_LRD_LAUNCH(3, D); break;       \
      default: FT_LRD_LAUNCH(4, D); break;      \
    }
    if (ndb == 1) { FT_LRD_SWITCH(1) } else { FT_LRD_SWITCH(2) }
#undef FT_LRD_SWITCH
  } else if (hout) {
    switch (nct) {
      case 0: FT_LRG_LAUNCH(0); break;
      case 1: FT_LRG_LAUNCH(1); break;
      case 2: FT_LRG_LAUNCH(2); break;
      case 3: FT_LRG_LAUNCH(3); break;
      default: FT_LRG_LAUNCH(4); break;
    }
  } else if (quant) {
    switch (nct) {
      case 0: FT_LR_LAUNCH(0, true); break;
      case 1: FT_LR_LAUNCH(1, true); break;
      case 2: FT_LR_LAUNCH(2, true); break;
      case 3: FT_LR_LAUNCH(3, true); break;
      default: FT_LR_LAUNCH(4, true); break;
    }
  } else {
    switch (nct) {
      case 1: FT_LR_LAUNCH(1, false); break;
      case 2: FT_LR_LAUNCH(2, false); break;
      case 3: FT_LR_LAUNCH(3, false); break;
      default: FT_LR_LAUNCH(4, false); break;
    }
  }
#undef FT_LR_LAUNCH
#undef FT_LRG_LAUNCH
#undef FT_LR_ANY
#undef FT_LR_ONE
#undef FT_LRD_LAUNCH
  if (launch_status() != FT_OK) return FT_EHIP;
  if (S > 1 && rho) {
    hipLaunchKernelGGL(sum_splits_kernel, dim3((unsigned)((stride / 4 + 255) / 256)), dim3(256), 0, stream,
                       static_cast<const float*>(workspace), S, stride, out);
    if (launch_status() != FT_OK) return FT_EHIP;
  }
  if (dbp) {   // dB = the row blocks' partials added in row-block order
    const int64_t n = (int64_t)db.r * Kin;
    hipLaunchKernelGGL(sum_splits_kernel, dim3((unsigned)((n / 4 + 255) / 256)), dim3(256), 0, stream,
                       static_cast<const float*>(db.part), row_blocks(M), n, dB);
    return launch_status();
  }
  return FT_OK;
}
}  // namespace
}  // namespace ft

extern "C" ft_status ft_lowrank_fused(const void* in, int64_t M, int64_t Kin, int64_t ld_in,
                                      const void* wa, int32_t ra, const void* wb, int32_t rb,
                                      float* out, void* workspace, size_t ws_bytes, hipStream_t stream) {
  return ft::lowrank_impl(in, M, Kin, ld_in, wa, ra, wb, rb, out, nullptr, nullptr, workspace, ws_bytes, stream);
}

extern "C" ft_status ft_lowrank_plan(int64_t M, int64_t Kin, int32_t rho, int32_t* plan) {
  using namespace ft;
  if (!plan) return FT_EINVAL;
  if (!mult16(M) || !mult16(Kin) || rho < 0 || rho % 16 || rho > 128) return FT_ESHAPE;
  if (M == 0 || Kin == 0) {
    for (int i = 0; i < 5; ++i) plan[i] = 0;
    return FT_OK;
  }
  const LrPlan pl = lowrank_plan(M, Kin, rho, false);
  plan[0] = LR_ROWS / pl.wc;
  plan[1] = pl.lines ? 1 : 0;
  plan[2] = (int32_t)pl.splits;
  plan[3] = (int32_t)pl.cps;
  plan[4] = (int32_t)pl.lds;
  return FT_OK;
}

extern "C" ft_status ft_quant_lowrank(const void* in, int64_t M, int64_t Kin, int64_t ld_in,
                                      const void* wa, int32_t ra, const void* wb, int32_t rb, float* out,
                                      uint8_t* codes_rm, uint8_t* scales, void* workspace, size_t ws_bytes,
                                      hipStream_t stream) {
  if (!codes_rm) return FT_EINVAL;
  return ft::lowrank_impl(in, M, Kin, ld_in, wa, ra, wb, rb, out, codes_rm, scales, workspace, ws_bytes, stream);
}

extern "C" ft_status ft_gelu_quant_lowrank(const void* y, int64_t M, int64_t Kin, const void* wa, int32_t ra,
                                           const void* wb, int32_t rb, void* h, float* out, uint8_t* codes_rm,
                                           uint8_t* scales, void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (!codes_rm || !scales || (M && Kin && !h)) return FT_EINVAL;
  if (Kin == 0 || M == 0) return ft::lowrank_impl(y, M, Kin, Kin, wa, ra, wb, rb, out, codes_rm, scales, workspace,
                                                  ws_bytes, stream);
  return ft::lowrank_impl(y, M, Kin, Kin, wa, ra, wb, rb, out, codes_rm, scales, workspace, ws_bytes, stream, h);
}

extern "C" size_t ft_quant_lowrank_db_workspace(int64_t M, int64_t Kin, int32_t rho, int32_t r) {
  using namespace ft;
  if (M <= 0 || Kin <= 0 || rho < 0 || r < 0) return 0;
  const size_t v = rho ? ft_lowrank_workspace(M, Kin, rho) : 0;
  return ((v + 255) & ~(size_t)255) + (size_t)row_blocks(M) * r * Kin * sizeof(float);
}

extern "C" ft_status ft_quant_lowrank_db(const void* g, int64_t M, int64_t N, int64_t ld_g, const void* L2, int32_t rs,
                                         const void* B, int32_t r, float* V, uint8_t* codes_rm, uint8_t* scales,
                                         const float* T, float* dB, void* workspace, size_t ws_bytes,
                                         hipStream_t stream) {
  using namespace ft;
  if (!codes_rm || !scales) return FT_EINVAL;
  if (r < 0 || r > 64 || r % 16 || rs < 0 || rs % 16 || rs + r > 128) return FT_ESHAPE;
  if (r == 0 || M == 0 || N == 0) {   // no adapter gradient to fold in (or an empty one)
    if (r && N && dB) {
      const ft_status z = fill_zero_f32(dB, (int64_t)r * N, stream);
      if (z != FT_OK) return z;
    }
    return lowrank_impl(g, M, N, ld_g, L2, rs, B, r, V, codes_rm, scales, workspace, ws_bytes, stream);
  }
  if (!T || !dB) return FT_EINVAL;
  if (!aligned16(T) || !aligned16(dB)) return FT_EALIGN;
  DbArgs db{T, (int64_t)(rs + r), rs, r, nullptr};
  return lowrank_impl(g, M, N, ld_g, L2, rs, B, r, V, codes_rm, scales, workspace, ws_bytes, stream, nullptr, &db,
                      dB);
}
