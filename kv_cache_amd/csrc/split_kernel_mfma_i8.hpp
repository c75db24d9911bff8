// Split kernel for the int8 K/V format with D = 128: QK^T and PV on the
// matrix cores.
//
// Format ("M8.6 - Live-Data Quantization: Activations and KV Cache",
// sections 0x06-0x06C): K codes with one fp16 scale per (128-token group,
// channel), V codes with one fp16 scale per token, and the newest min(T, R)
// tokens as bf16 rows; quantized history and residual share one softmax.
//
// A workgroup's visible ordinals [begin, end) split into an int8 part
// [begin, mid) and a residual part [mid, end) (positions grow with the
// ordinal and the residual holds the newest positions).  Both parts run the
// tile loop of split_kernel_mfma with the same running state:
//
//  * int8 part.  A per-channel K scale cannot leave the dot product (section
//    0x03B), so each K element is dequantized inside the reduction: the code
//    becomes an exact fp16 value (bias 1024+128 trick: the byte c^0x80 is the
//    mantissa of 1024 + (c + 128)), is multiplied by its fp16 channel scale in
//    packed fp16 arithmetic as an unevaluated sum hi + lo (exact to 2^-22),
//    and both parts feed v_mfma_f32_16x16x32_f16 with q in fp16 (B operand).  Each row reads its
//    own 128-token group's scales (staged in LDS per phase of the split), so
//    groups never need special handling.  The V scale of a row multiplies
//    that row's softmax weight (section 0x03C) before PV, which runs on
//    v_mfma_f32_16x16x32_f16 with the V codes as exact fp16 subnormals
//    (c + 128) * 2^-24 (one v_perm per pair) and removes the 128 * sum(weights)
//    bias with one more MFMA against a constant; the denominator uses the
//    unscaled weight.  Each wave keeps two tiles in flight.
//  * residual part: exactly the bf16 kernel's tile (A = bf16 K rows, B = q).
#pragma once

#include "split_kernel_mfma.hpp"

namespace da {

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

// Round two floats to fp16 (nearest even) and pack them, first in the low half.
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}

// Eight int8 codes times their eight fp16 scales as fp16 pairs hi + lo with
// hi = fp16(c * sigma) and lo = fp16(c * sigma - hi) (the fused multiply-add
// forms c * sigma - hi exactly, and c * sigma has at most 18 significant bits,
// so hi + lo represents the product to 2^-22).  Codes: the byte c ^ 0x80 =
// c + 128 placed under the exponent of 1024 gives the fp16 value
// 1024 + c + 128 exactly; subtracting 1152 leaves c exactly.
__device__ __forceinline__ void dequant_f16(uint2 codes, uint4 scales, uint4& hi, uint4& lo) {
  const uint32_t w[2] = {codes.x ^ 0x80808080u, codes.y ^ 0x80808080u};
  const uint32_t sc[4] = {scales.x, scales.y, scales.z, scales.w};
  uint32_t oh[4], ol[4];
  const f16x2_t bias = {(_Float16)1152.0f, (_Float16)1152.0f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // code bytes 2(i&1) and 2(i&1)+1 of word i/2 under the exponent byte 0x64
    const uint32_t sel = (uint32_t)(2 * (i & 1)) | 0x0400u | ((uint32_t)(2 * (i & 1) + 1) << 16) | 0x04000000u;
    const uint32_t bits = __builtin_amdgcn_perm(0x64646464u, w[i >> 1], sel);
    const f16x2_t c = __builtin_bit_cast(f16x2_t, bits) - bias;
    const f16x2_t sg = __builtin_bit_cast(f16x2_t, sc[i]);
    const f16x2_t h = c * sg;
    oh[i] = __builtin_bit_cast(uint32_t, h);
    ol[i] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(c, sg, -h));
  }
  hi = make_uint4(oh[0], oh[1], oh[2], oh[3]);
  lo = make_uint4(ol[0], ol[1], ol[2], ol[3]);
}

// V codes of channel e (0..7) of two rows a, b as one fp16 pair of exact
// subnormals ((c_a[e] + 128) * 2^-24, (c_b[e] + 128) * 2^-24): the code words
// arrive with every byte xor 0x80 (so a byte is c + 128, in [1, 255]) and
// v_perm places the two bytes under zero bytes, the fp16 subnormal whose
// mantissa is the byte.  PV over these values is 2^-24 (sum w c + 128 sum w);
// the bias term is accumulated beside it and removed at the end.
__device__ __forceinline__ uint32_t v_pair_biased(uint2 a, uint2 b, int e) {
  const uint32_t wa = e < 4 ? a.x : a.y, wb = e < 4 ? b.x : b.y;
  const uint32_t sel = (uint32_t)(e & 3) | 0x0C00u | ((uint32_t)(4 + (e & 3)) << 16) | 0x0C000000u;
  return __builtin_amdgcn_perm(wb, wa, sel);
}
// 128 * 2^-24 = 2^-17 as an fp16 subnormal pair: the B operand of the bias term
constexpr uint32_t kVBiasPair = 0x00800080u;

// Largest magnitude bit pattern (sign cleared) of the eight 16-bit floats
// (fp16 or bf16: ordering by magnitude is ordering of these bits) in x.
__device__ __forceinline__ uint32_t f16_absmax_bits(uint4 x) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) m = max(m, max(w[i] & 0x7fffu, (w[i] >> 16) & 0x7fffu));
  return m;
}
// The eight fp16 values of x times 2^-e (exact while the results stay normal).
__device__ __forceinline__ uint4 f16_scale_pow2(uint4 x, int e) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
  uint32_t r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    r[i] = pack_f16(ldexpf(f16_bits_to_f32(w[i] & 0xffffu), -e), ldexpf(f16_bits_to_f32(w[i] >> 16), -e));
  return make_uint4(r[0], r[1], r[2], r[3]);
}
// Wave-wide maximum (wave-uniform result): DPP inside each 16-lane row, then
// the four row maxima read into scalar registers.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, dpp_u32<0xB1>(x));    // quad_perm [1,0,3,2]
  x = max(x, dpp_u32<0x4E>(x));    // quad_perm [2,3,0,1]
  x = max(x, dpp_u32<0x141>(x));   // row_half_mirror
  x = max(x, dpp_u32<0x140>(x));   // row_mirror
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)x, 0), b = (uint32_t)__builtin_amdgcn_readlane((int)x, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)x, 32), d = (uint32_t)__builtin_amdgcn_readlane((int)x, 48);
  return max(max(a, b), max(c, d));
}
// floor(log2 x) of a normal fp16 magnitude bit pattern (subnormals: -14)
__device__ __forceinline__ int f16_exponent(uint32_t bits) { return max((int)(bits >> 10), 1) - 15; }

// a * b for a, b < 2^24 with a product below 2^32 (v_mul_u32_u24), unsigned so
// that it extends to an address offset by zero extension
__device__ __forceinline__ uint32_t mul_u24(uint32_t a, uint32_t b) { return (uint32_t)__umul24(a, b); }

// K scale rows staged in LDS per workgroup (256 B each for D = 128): a phase
// of at most 23 groups' length starting anywhere in a group touches at most
// 24 of them.  A phase is at most kI8PhaseRows rows (the V-scale pre-pass of
// a phase start reads 12 scales per lane: 3072 rows over the 4 waves' tiles).
constexpr int kI8ScaleSlots = 24;
constexpr int kI8PhaseRows = 3072;

// A partitioned run keeps the state of several pieces' walk live: it gets
// the register budget of 2 waves per SIMD, and the host sizes its default
// partition for 2 workgroups per CU.
constexpr int kI8PartitionWgPerCu = 2;

// 3 waves per SIMD (<= 168 VGPRs) up to 4 heads per group, 2 for 8 heads;
// OCC2: the instance for grids of at most 2 workgroups per CU, with the
// register budget of 2 waves per SIMD (<= 256 VGPRs).
// INSTR: kInstrRows is the index-trace instance, which also records each row
// load (codes, scales, residual rows) where it is issued; kInstrStamps
// records per-workgroup timestamps; otherwise identical.  PART: the balanced
// partition instance (workgroup (item, h_kv) runs the request pieces of its
// item, as in split_kernel_mfma).
template <int G, int NWAVES, bool FUSED, int INSTR = 0, bool PART = false, bool OCC2 = false>
__global__ __launch_bounds__(NWAVES * 64, PART ? kI8PartitionWgPerCu : (G <= 4 && !OCC2 ? 3 : 2)) void split_kernel_mfma_i8(SplitParams p) {
  constexpr int D = 128;
  // The sink tile (below) keeps another tile's registers live at a phase
  // start: only instances with the 2-waves-per-SIMD budget take it.
  constexpr bool kMergeSinks = PART || OCC2 || G > 4;
  constexpr int TW = 16;
  constexpr int STEP = NWAVES * TW;
  static_assert(G >= 1 && G <= 16, "");

  WgStamps<INSTR> stamps(p);
  const PartitionHeaderAtExit header_at_exit{p};
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform (SGPR)
  const int n = lane & 15;     // K row of the tile / score column (head)
  const int kg = lane >> 4;    // channel group of the MFMA slice / V row slot
  __shared__ uint4 q_lds[4][64];
  __shared__ uint4 ksc[NWAVES][kI8ScaleSlots][16];   // one K scale table per wave
  __shared__ WaveStates<G, D, NWAVES> sh;

  // One piece of work: visible ordinals [pbeg, pend) of request b for K/V
  // head h, stored as split slot s.  pend < 0: the plan's split s.
  auto piece = [&](int b, int h, int s, int pbeg, int pend) {
  // The request length is requested first, so its round trip overlaps the
  // q staging below instead of following its barrier.
  const int T = request_len(p, b);
  // q rows in the B operand layout, q[head n][32c + 8kg .. +7] (zero for
  // n >= G), staged in LDS: the residual part uses them as they are, the int8
  // part reads them in its own channel order.
  if (wave == 0) {
    // all four loads in flight at once (lanes n >= G read head 0's row and
    // store zeros), so the staging costs one round trip
    const uint16_t* qrow = static_cast<const uint16_t*>(p.q) + out_row(p, b, h, n < G ? n : 0) * D + 8 * kg;
    uint4 x[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) x[c] = *reinterpret_cast<const uint4*>(qrow + 32 * c);
#pragma unroll
    for (int c = 0; c < 4; ++c) q_lds[c][lane] = n < G ? x[c] : make_uint4(0u, 0u, 0u, 0u);
  }
  __syncthreads();

  const VisProgram vis = make_vis(T, p.mask_kind, p.n_sink, p.window);
  const int n_q = quantized_len(p, T);
  const int o_res = residual_ordinal(vis, n_q);
  int begin, end;
  if (pend < 0) {
    split_range_weighted(vis.n_vis, o_res, s, p.chunk, &begin, &end);
  } else {
    begin = min(pbeg, vis.n_vis);
    end = min(pend, vis.n_vis);
  }
  // Score column n is virtual head n, with its own visible end (C > 1 rows).
  const int lim_n = row_limit(p, vis.n_vis, n);
  if (begin >= end) {
    write_identity<G, D, NWAVES, FUSED>(p, b, h, s);
    stamps.states_stored();
    stamps.folded = finish_split<G, D, NWAVES, FUSED>(p, b, h);
    return;
  }
  const int mid = min(max(o_res, begin), end);

  const uint32_t row_stride = (uint32_t)(p.num_kv_heads * D);
  const int64_t code_base = ((int64_t)b * p.kv_capacity * p.num_kv_heads + h) * D;
  const int8_t* kc = static_cast<const int8_t*>(p.k) + code_base;
  const int8_t* vc = static_cast<const int8_t*>(p.v) + code_base;
  const int64_t res_base = ((int64_t)b * p.residual_len * p.num_kv_heads + h) * D;
  const uint16_t* kr = static_cast<const uint16_t*>(p.k_resid) + res_base + 8 * kg;
  const uint16_t* vr = static_cast<const uint16_t*>(p.v_resid) + res_base + 8 * n;
  const int n_groups = (p.kv_capacity + (1 << p.k_group_shift) - 1) >> p.k_group_shift;
  const int64_t ks_base = ((int64_t)b * n_groups * p.num_kv_heads + h) * D;
  const int64_t vs_base = (int64_t)b * p.kv_capacity * p.num_kv_heads + h;
  const uint16_t* ks = p.k_scale + ks_base;
  const uint16_t* vs = p.v_scale + vs_base;

  float m_run = -INFINITY;   // running max of head n (base 2)
  float l_run = 0.f;         // partial denominator over rows 4kg .. 4kg+3 of every tile
  // fp16 range of the int8 part's matrix-core operands.  Each operand is
  // brought into range by a power of two that the scores or the weights undo
  // exactly, per wave and per phase of the split, where it needs it:
  //  * q per head, when its largest |q| is below 2^-4 or 2^15 or more: into
  //    [2^14, 2^15) (q * 2^-e_q);
  //  * the phase's K scale rows, when their largest scale is 2^9 or more:
  //    into [2^8, 2^9) (times 2^-e_k), so code * scale < 2^16;
  //  * the V scales of the wave's rows of the phase, when their largest is
  //    below 2^-3: into [2^14, 2^15) (times 2^-e_v), so small scales do not
  //    fall to fp16 subnormals (weight * scale never exceeds the scale).
  // Scores are acc * sfac with sfac = scale * log2(e) * 2^(e_q + e_k); the
  // weights p * sigma_V enter PV times vinv = 2^-e_v (the denominator takes
  // p), so o holds u * 2^-e_v and is multiplied by vpow = 2^e_v at the end.
  float sfac = p.qscale;
  int e_v = 0;
  float vpow = 1.f, vinv = 1.f;
  f32x4_t o[8];              // int8 part: PV accumulators in the matrix-core layout
#pragma unroll
  for (int c = 0; c < 8; ++c) o[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // 2^-17 * (sum of the weights) per head, in o's layout (every channel
  // block carries the same bias term); o - obias is 2^-24 * u
  f32x4_t obias = {0.f, 0.f, 0.f, 0.f};

  // Online softmax over the 8 scores of this lane for two tiles (rows
  // 4kg+i of tiles ta and tb, head n).
  auto softmax2 = [&](const f32x4_t& acc, const f32x4_t& acc2, int ta, int tb, int lim, float (&pr)[8]) -> float {
    float sc[8];
    const int l = min(lim, lim_n);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sc[i] = (ta + 4 * kg + i < l) ? acc[i] * sfac : -INFINITY;
      sc[4 + i] = (tb + 4 * kg + i < l) ? acc2[i] * sfac : -INFINITY;
    }
    float mt = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])),
                     fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
    mt = xor32_max(xor16_max(mt));
    const float mn = fmaxf(m_run, mt);
    const float mz = mn == -INFINITY ? 0.f : mn;
    const float alpha = fast_exp2(m_run - mz);
#pragma unroll
    for (int i = 0; i < 8; ++i) pr[i] = fast_exp2(sc[i] - mz);
    l_run = fmaf(l_run, alpha, ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7])));
    m_run = mn;
    return alpha;
  };

  // ================= int8 part: ordinals [begin, mid) =================
  // K codes.  Lane (n, kg) holds 32 codes of row n of the tile: bytes
  // [16kg, 16kg+16) and [64+16kg, 64+16kg+16), so each of the two 16-byte
  // requests covers 64 contiguous bytes of every row (half a cache line)
  // instead of 32-byte quarters.  Its MFMA slice c then carries the channels
  // kch(c) .. kch(c)+7 below; q and the scales are read in the same order,
  // which leaves every dot product unchanged (it is a sum over channels).
  //
  // Scales.  The K scale rows of the 128-token groups a phase of the split
  // touches are staged in LDS; a phase is short enough for the table, so a
  // tile in flight holds only codes and V scales and each wave keeps two
  // tiles in flight.  A split is one phase per run unless it is long.
  auto kch = [&](int c) { return 64 * (c >> 1) + 16 * kg + 8 * (c & 1); };
  if (begin < mid) {
    // q in this part's channel order, read from the staged rows: channels
    // kch(c) .. +7 of head n are 8-channel block kch(c)/8 = 4c' + kg', held by
    // lane n + 16kg' of q_lds[c'] (zero for n >= G).
    // Head n's largest |q| (bf16 bit pattern, read by each of its lanes from
    // all 16 staged blocks, so the four lanes of a head agree) sets e_q, and
    // q * 2^-e_q (exact in fp16 down to 2^-28 of the largest) feeds the
    // matrix cores.
    uint32_t qmx = 0;
#pragma unroll
    for (int blk = 0; blk < 16; ++blk) qmx = max(qmx, f16_absmax_bits(q_lds[blk >> 2][n + 16 * (blk & 3)]));
    // (bf16 exponent of the largest |q|; q of magnitude in [2^-4, 2^15) is
    // used as it is)
    const int eq_max = (int)(qmx >> 7) - 127;
    const int e_q = (qmx == 0 || (eq_max >= -4 && eq_max < 15)) ? 0 : min(max(eq_max - 14, -100), 100);
    uint4 qh[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int blk = kch(c) >> 3;
      const uint4 x = q_lds[blk >> 2][n + 16 * (blk & 3)];
      auto cv = [&](uint32_t wd) {
        return pack_f16(ldexpf(bf16_lo(wd), -e_q), ldexpf(bf16_hi(wd), -e_q));
      };
      qh[c] = make_uint4(cv(x.x), cv(x.y), cv(x.z), cv(x.w));
    }
    const int sh = p.k_group_shift;
    // Ordinals map to positions by a constant shift inside each run (sinks:
    // 0, window: gap), so a phase never spans the seam: its rows are the
    // positions t_pb + r, r in [0, pe - pb), addressed from wave-uniform bases
    // with unsigned lane offsets r * row_stride formed by 24-bit multiplies
    // (r < kI8PhaseRows = 3072 and row_stride <= 2^20 bytes keep them below
    // 2^32).  A phase of at most (slots - 2) groups' length touches at most
    // `slots - 1` scale rows (the last slot holds the sink tile's row, below).
    // Every phase start costs one round trip to memory (its scale rows), so
    // phases are as long as the table allows.
    const int phase = min((kI8ScaleSlots - 2) << sh, kI8PhaseRows);
    const uint32_t vs_stride = 2 * (uint32_t)p.num_kv_heads;   // V scale bytes per position
    // Sink tile: when the split's sink ordinals [s_b, s_e) fit one tile
    // inside one K group and the split also has int8 window rows, wave 0
    // takes the sinks as one extra tile of the first window phase (their K
    // scale row in the table's last slot, their V scales in the wave's
    // normalization), so the split pays one phase start instead of two.
    const int s_b = begin, s_e = min(mid, vis.ns), w_b = max(begin, vis.ns);
    const bool sink_tile = kMergeSinks && s_b < s_e && w_b < mid && s_e - s_b <= TW &&
                           (s_b >> sh) == ((s_e - 1) >> sh);
    constexpr int kSinkSlot = kI8ScaleSlots - 1;
    for (int run = sink_tile ? 1 : 0; run < 2; ++run) {
      const int rb = run == 0 ? begin : max(begin, vis.ns);
      const int re = run == 0 ? min(mid, vis.ns) : mid;
      const int shift = run == 0 ? 0 : vis.gap;
      for (int pb = rb; pb < re; pb += phase) {
        const int pe = min(pb + phase, re);
        const int t_pb = pb + shift;
        const int g0 = t_pb >> sh;
        const int ng = ((pe - 1 + shift) >> sh) - g0 + 1;
        const int8_t* kp = kc + (uint64_t)t_pb * row_stride;
        const int8_t* vp = vc + (uint64_t)t_pb * row_stride;
        const char* vsp = reinterpret_cast<const char*>(vs + (int64_t)t_pb * p.num_kv_heads);
        const uint32_t last = (uint32_t)(pe - 1 - pb);
        // row of ordinal o within the phase, clamped to its last row
        auto rel = [&](int o) { return min((uint32_t)(o - pb), last); };
        auto slot = [&](int tile) { return (int)((t_pb + rel(tile + n)) >> sh) - g0; };
        auto issue_k = [&](int tile, uint4 (&k)[2]) {
          const uint32_t off = mul_u24(rel(tile + n), row_stride) + 16 * kg;
          k[0] = stream_load<kHalfLineNT>(reinterpret_cast<const uint4*>(kp + off));
          k[1] = stream_load<kHalfLineNT>(reinterpret_cast<const uint4*>(kp + off + 64));
          if constexpr (INSTR == kInstrRows) {
            // the row's codes, and the scale row its dequantization reads
            // (staged from k_scale row g0 + slot)
            if (kg == 0 && tile + n < pe)
              trace_k(p, b, h, tile + n, t_pb + (int)rel(tile + n),
                      code_base + (int64_t)t_pb * row_stride + (off - 16 * kg),
                      ks_base + (int64_t)(g0 + slot(tile)) * row_stride);
          }
        };
        // V rows 4kg + j of the tile, and one V scale per lane: lane (n, kg)
        // with n < 4 reads the scale of row 4kg + n, which PV broadcasts
        // across its 16-lane row (row_newbcast:j gives row 4kg + j); the other
        // lanes repeat a row of theirs.
        auto issue_v = [&](int tile, uint2 (&v)[4], uint32_t& sv) {
          sv = *reinterpret_cast<const uint16_t*>(vsp + mul_u24(rel(tile + 4 * kg + (n & 3)), vs_stride));
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t r = rel(tile + 4 * kg + j);
            v[j] = stream_load(reinterpret_cast<const uint2*>(vp + (mul_u24(r, row_stride) + 8 * (uint32_t)n)));
            if constexpr (INSTR == kInstrRows) {
              if (n == 0 && tile + 4 * kg + j < pe)
                trace_v(p, b, h, tile + 4 * kg + j, code_base + (int64_t)t_pb * row_stride + mul_u24(r, row_stride),
                        vs_base + (int64_t)t_pb * p.num_kv_heads + mul_u24(r, vs_stride) / 2);
            }
          }
        };
        auto scores_sl = [&](int sl, const uint4 (&k)[2]) {
          f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const uint4 w = k[c >> 1];
            const uint2 codes = (c & 1) ? make_uint2(w.z, w.w) : make_uint2(w.x, w.y);
            uint4 hi, lo;
            dequant_f16(codes, ksc[wave][sl][kch(c) >> 3], hi, lo);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, hi),
                                                         __builtin_bit_cast(f16x8_t, qh[c]), acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, lo),
                                                         __builtin_bit_cast(f16x8_t, qh[c]), acc, 0, 0, 0);
          }
          return acc;
        };
        auto scores = [&](int tile, const uint4 (&k)[2]) { return scores_sl(slot(tile), k); };
        // PV on the matrix cores, O (heads x channels) += P (heads x rows) V
        // (rows x channels) over the 32 rows of the two tiles: A = the weights
        // p * sigma_V in fp16 (relative error 2^-11, far inside the int8 format's
        // own error; lane (n, kg) already holds head n's weights of rows 4kg..4kg+3
        // of both tiles, the A operand's k = 8kg .. 8kg+7), B = the V codes as
        // exact fp16, whose lane (n, kg) holds the same rows at 8 channels 8n ..
        // 8n+7: instruction c takes channel 8n + c of each row, so column n of
        // block c is channel 8n + c and no code moves between lanes.  The
        // accumulator o[c] of lane (n, kg) holds heads 4kg .. 4kg+3 at channel
        // 8n + c.  The denominator uses the unscaled weights.
        auto pv2 = [&](const uint2 (&a)[4], uint32_t sa, const uint2 (&bv)[4], uint32_t sb,
                       const float (&pr)[8]) {
          uint4 w;
          float ps[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) ps[i] = pr[i] * vinv;
          // scale of row 4kg + j: lane j of this lane's 16-lane row
          auto sc = [](uint32_t x, auto J) {
            return f16_bits_to_f32((uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x150 + decltype(J)::value,
                                                                          0xF, 0xF, false));
          };
          using J0 = std::integral_constant<int, 0>;
          using J1 = std::integral_constant<int, 1>;
          using J2 = std::integral_constant<int, 2>;
          using J3 = std::integral_constant<int, 3>;
          w.x = pack_f16(ps[0] * sc(sa, J0{}), ps[1] * sc(sa, J1{}));
          w.y = pack_f16(ps[2] * sc(sa, J2{}), ps[3] * sc(sa, J3{}));
          w.z = pack_f16(ps[4] * sc(sb, J0{}), ps[5] * sc(sb, J1{}));
          w.w = pack_f16(ps[6] * sc(sb, J2{}), ps[7] * sc(sb, J3{}));
          uint2 ax[4], bx[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            ax[j] = make_uint2(a[j].x ^ 0x80808080u, a[j].y ^ 0x80808080u);
            bx[j] = make_uint2(bv[j].x ^ 0x80808080u, bv[j].y ^ 0x80808080u);
          }
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            const uint4 vcol = make_uint4(v_pair_biased(ax[0], ax[1], c), v_pair_biased(ax[2], ax[3], c),
                                          v_pair_biased(bx[0], bx[1], c), v_pair_biased(bx[2], bx[3], c));
            o[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, w),
                                                          __builtin_bit_cast(f16x8_t, vcol), o[c], 0, 0, 0);
          }
          const uint4 kb4 = make_uint4(kVBiasPair, kVBiasPair, kVBiasPair, kVBiasPair);
          obias = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, w),
                                                         __builtin_bit_cast(f16x8_t, kb4), obias, 0, 0, 0);
        };
        // running-maximum rescale of o: lane (n, kg) scales heads 4kg .. 4kg+3
        auto rescale_o = [&](float alpha) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float a = __shfl(alpha, 4 * kg + i);
#pragma unroll
            for (int c = 0; c < 8; ++c) o[c][i] *= a;
            obias[i] *= a;
          }
        };
        // Phase start, per wave (no workgroup barrier): the wave stages its own
        // copy of the phase's K scale rows and finds the largest K scale of
        // the phase and the largest V scale of its own rows, which set its
        // e_k and e_v (see above).  The scale loads are issued first and the
        // first tiles after them (addresses clamped into the phase, so all
        // loads are unconditional), so the scales, returned first, are reduced
        // and staged while the tiles are in flight.  Duplicates from clamping
        // change no maximum.
        // K scale quads idx = lane + 64k of the phase's rows, all requested
        // here (clamped: a phase touches at most kI8ScaleSlots rows of 16 quads)
        constexpr int kKq = kI8ScaleSlots * 16 / 64;
        uint4 kq[kKq];
#pragma unroll
        for (int k = 0; k < kKq; ++k) {
          const int i = min(lane + 64 * k, ng * 16 - 1);
          kq[k] = *reinterpret_cast<const uint4*>(ks + (uint64_t)(g0 + (i >> 4)) * row_stride + 8 * (i & 15));
        }
        // this wave's rows: tiles pb + 16*wave + 64k, 16 rows each; lane l
        // takes row 16*wave + 64*(4j + l/16) + l%16 of the phase for load j
        uint32_t vsv[kI8PhaseRows / 256];
#pragma unroll
        for (int j8 = 0; j8 < kI8PhaseRows / 256; ++j8) {
          const uint32_t r = min((uint32_t)(16 * wave + 64 * (4 * j8 + (lane >> 4)) + (lane & 15)), last);
          vsv[j8] = *reinterpret_cast<const uint16_t*>(vsp + mul_u24(r, vs_stride));
        }
        // The sink tile (wave 0 of the first window phase): its K scale row
        // (lanes 0..15), codes and V scales, requested before the phase's tiles.
        const bool sink_here = sink_tile && run == 1 && pb == w_b && wave == 0;   // wave-uniform
        uint4 kqs = make_uint4(0u, 0u, 0u, 0u), sk[2];
        uint2 sv4[4];
        uint32_t svs = 0;
        if (sink_here) {
          if (lane < 16) kqs = *reinterpret_cast<const uint4*>(ks + (uint64_t)(s_b >> sh) * row_stride + 8 * lane);
          const uint32_t rk = (uint32_t)min(s_b + n, s_e - 1);
          const uint32_t rs = (uint32_t)min(s_b + 4 * kg + (n & 3), s_e - 1);
          svs = *reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(vs) + (uint64_t)rs * vs_stride);
          sk[0] = stream_load<kHalfLineNT>(reinterpret_cast<const uint4*>(kc + (uint64_t)rk * row_stride + 16 * kg));
          sk[1] = stream_load<kHalfLineNT>(reinterpret_cast<const uint4*>(kc + (uint64_t)rk * row_stride + 64 + 16 * kg));
          if constexpr (INSTR == kInstrRows) {
            if (kg == 0 && s_b + n < s_e)
              trace_k(p, b, h, s_b + n, s_b + n, code_base + (int64_t)rk * row_stride,
                      ks_base + (int64_t)(s_b >> sh) * row_stride);
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t rv = (uint32_t)min(s_b + 4 * kg + j, s_e - 1);
            sv4[j] = stream_load(reinterpret_cast<const uint2*>(vc + (uint64_t)rv * row_stride + 8 * (uint32_t)n));
            if constexpr (INSTR == kInstrRows) {
              if (n == 0 && s_b + 4 * kg + j < s_e)
                trace_v(p, b, h, s_b + 4 * kg + j, code_base + (int64_t)rv * row_stride,
                        vs_base + (int64_t)rv * p.num_kv_heads);
            }
          }
        }
        uint4 ka[2], kb[2];
        uint2 va[4], vb[4];
        uint32_t sva, svb;
        // Sweep order: the phase's pairs of steps (wave w takes tiles w and
        // w + NWAVES of each pair) are visited from pair q0 on and wrap around,
        // q0 staggering requests and splits (sweep_start; K/V codes of equal
        // requests lie a power of two apart); the requests after the last pair
        // repeat the phase's last row.
        const int n_pairs = (pe - pb + 2 * STEP - 1) / (2 * STEP);
        const int n_mine = max(0, (pe - pb - wave * TW + 2 * STEP - 1) / (2 * STEP));   // pairs with a tile of this wave
        int q0 = sweep_start(b, s, n_pairs);
        if (q0 >= n_mine) q0 = 0;
        auto pair_tile = [&](int k) -> int {
          if (k >= n_mine) return pe + wave * TW;
          const int q = q0 + k;
          return pb + 2 * STEP * (q >= n_mine ? q - n_mine : q) + wave * TW;
        };
        int tile = pair_tile(0);
        // the loop's request order (K, K, V, V), so its waits leave newer requests in flight
        issue_k(tile, ka);
        issue_k(tile + STEP, kb);
        issue_v(tile, va, sva);
        issue_v(tile + STEP, vb, svb);
        uint32_t kmx = 0, vmx = 0;
#pragma unroll
        for (int k = 0; k < kKq; ++k) {
          kmx = max(kmx, f16_absmax_bits(kq[k]));
          const int idx = lane + 64 * k;
          if (idx < ng * 16) ksc[wave][idx >> 4][idx & 15] = kq[k];
        }
#pragma unroll
        for (int j8 = 0; j8 < kI8PhaseRows / 256; ++j8) vmx = max(vmx, vsv[j8] & 0x7fffu);
        if (sink_here) {
          kmx = max(kmx, f16_absmax_bits(kqs));        // lanes >= 16 hold zeros
          vmx = max(vmx, svs & 0x7fffu);
          if (lane < 16) ksc[0][kSinkSlot][lane] = kqs;
        }
        kmx = wave_max_u32(kmx);
        vmx = wave_max_u32(vmx);
        // K rows are scaled only where code * scale could reach fp16's range
        const int e_k = max(f16_exponent(kmx) - 8, 0);
        // V scales of 2^-3 or more need no scaling: weights below fp16's
        // normal range then carry at most 2^-10 of the output
        const int e_v_new = f16_exponent(vmx) >= -3 ? 0 : f16_exponent(vmx) - 14;
        // the wave reads its table only after all of its lanes have written it
        auto wave_lds_sync = [] {
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the table stores have completed
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        };
        wave_lds_sync();
        if (e_k > 0) {               // rare: the table times 2^-e_k, in place
          for (int idx = lane; idx < ng * 16; idx += 64)
            ksc[wave][idx >> 4][idx & 15] = f16_scale_pow2(ksc[wave][idx >> 4][idx & 15], e_k);
          if (sink_here && lane < 16) ksc[0][kSinkSlot][lane] = f16_scale_pow2(ksc[0][kSinkSlot][lane], e_k);
          wave_lds_sync();
        }
        sfac = ldexpf(p.qscale, e_q + e_k);
        if (e_v_new != e_v) {        // o to the new units (o is 0 before the first phase)
          const float f = ldexpf(1.f, e_v - e_v_new);
#pragma unroll
          for (int c = 0; c < 8; ++c) o[c] *= f;
          obias *= f;
          e_v = e_v_new;
          vpow = ldexpf(1.f, e_v);
          vinv = ldexpf(1.f, -e_v);
        }
        if (sink_here) {
          // one tile of sink rows (the second tile of the pair is empty: its
          // ordinals start at s_e, all masked, weight 0)
          const f32x4_t acc = scores_sl(kSinkSlot, sk);
          float pr[8];
          const float alpha = softmax2(acc, acc, s_b, s_e, s_e, pr);
          if (__any(alpha != 1.f)) rescale_o(alpha);
          pv2(sv4, svs, sv4, svs, pr);
        }
        for (int k = 0; k < n_mine; ++k) {
          const int tb = tile + STEP;
          const int next = pair_tile(k + 1);
          const f32x4_t acc = scores(tile, ka);
          const f32x4_t acc2 = scores(tb, kb);
          issue_k(next, ka);
          issue_k(next + STEP, kb);
          float pr[8];
          const float alpha = softmax2(acc, acc2, tile, tb, pe, pr);
          if (__any(alpha != 1.f)) rescale_o(alpha);   // skipped while no head maximum moves
          pv2(va, sva, vb, svb, pr);
          issue_v(next, va, sva);
          issue_v(next + STEP, vb, svb);
          tile = next;
        }
      }
    }
  }

  // u in the vector-ALU layout of the residual part and the state merge: lane
  // (n, kg) holds a partial sum of head i at channels 8n .. 8n+7 (the partials
  // of the four kg lanes add up); head i of o sits in the kg = i/4 lanes.
  float u[G][8];
#pragma unroll
  for (int i = 0; i < G; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) u[i][e] = kg == (i >> 2) ? (o[e][i & 3] - obias[i & 3]) * (vpow * 16777216.f) : 0.f;

  // Online softmax over the 4 scores of this lane (rows 4kg+i, head n);
  // returns the weights and rescales l and u.
  auto softmax = [&](const f32x4_t& acc, int tile, int lim, float (&pr)[4]) {
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[i] = (tile + 4 * kg + i < min(lim, lim_n)) ? acc[i] * p.qscale : -INFINITY;
    float mt = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mt = xor32_max(xor16_max(mt));
    const float mn = fmaxf(m_run, mt);
    const float mz = mn == -INFINITY ? 0.f : mn;
    const float alpha = fast_exp2(m_run - mz);
#pragma unroll
    for (int i = 0; i < 4; ++i) pr[i] = fast_exp2(sc[i] - mz);
    l_run = fmaf(l_run, alpha, (pr[0] + pr[1]) + (pr[2] + pr[3]));
    m_run = mn;
    if (__any(alpha != 1.f)) HeadLoop<G>::rescale(u, alpha);   // skipped while no head max moved
  };

  // ============ residual part: ordinals [mid, end), bf16 rows ============
  if (mid < end) {
    auto rrow = [&](int o) { return (uint32_t)(vis_pos(vis, min(o, end - 1)) - n_q); };
    auto issue_k = [&](int tile, uint4 (&k)[4]) {
      const uint16_t* row = kr + (uint64_t)rrow(tile + n) * row_stride;
#pragma unroll
      for (int c = 0; c < 4; ++c) k[c] = stream_load<kHalfLineNT>(reinterpret_cast<const uint4*>(row + 32 * c));
      if constexpr (INSTR == kInstrRows) {
        if (kg == 0 && tile + n < end)
          trace_k(p, b, h, tile + n, vis_pos(vis, tile + n),
                  res_base + (int64_t)((uint64_t)rrow(tile + n) * row_stride));
      }
    };
    auto issue_v = [&](int tile, uint4 (&v)[4]) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[j] = stream_load(reinterpret_cast<const uint4*>(vr + (uint64_t)rrow(tile + 4 * kg + j) * row_stride));
        if constexpr (INSTR == kInstrRows) {
          if (n == 0 && tile + 4 * kg + j < end)
            trace_v(p, b, h, tile + 4 * kg + j,
                    res_base + (int64_t)((uint64_t)rrow(tile + 4 * kg + j) * row_stride));
        }
      }
    };
    MfmaTile t;
    int tile = mid + wave * TW;
    if (tile < end) {
      issue_k(tile, t.k);
      issue_v(tile, t.v);
    }
    for (; tile < end; tile += STEP) {
      const int next_tile = tile + STEP;
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, t.k[c]),
                                                      __builtin_bit_cast(bf16x8_t, q_lds[c][lane]), acc, 0, 0, 0);
      issue_k(next_tile, t.k);
      float pr[4];
      softmax(acc, tile, end, pr);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w[4] = {t.v[j].x, t.v[j].y, t.v[j].z, t.v[j].w};
        float vx[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) { vx[2 * e] = bf16_lo(w[e]); vx[2 * e + 1] = bf16_hi(w[e]); }
        HeadLoop<G>::accumulate(u, pr[j], vx);
      }
      issue_v(next_tile, t.v);
    }
  }

  // ---- wave state: all rows of a head share m, so l and u just add ---------
  l_run = xor32_sum(xor16_sum(l_run));
#pragma unroll
  for (int i = 0; i < G; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      u[i][e] = xor32_sum(xor16_sum(u[i][e]));
    }
  if (kg == 0) {
#pragma unroll
    for (int i = 0; i < G; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) sh.u[wave][i][8 * n + e] = u[i][e];
    if (n < G) {
      sh.m[wave][n] = m_run;
      sh.l[wave][n] = l_run;
    }
  }
  __syncthreads();
  merge_waves_and_store<G, D, NWAVES, FUSED>(p, b, h, s, sh);
  stamps.states_stored();
  stamps.folded = finish_split<G, D, NWAVES, FUSED>(p, b, h);
  };

  if constexpr (!PART) {
    int b, h, s;
    decode_workgroup(p, &b, &h, &s);
    piece(b, h, s, 0, -1);
  } else {
    // Balanced partition: workgroup (item, h) takes ordinals [item*L,
    // (item+1)*L) of the requests' visible ordinals laid end to end, one piece
    // per request it meets, stored as split slot (items since the request's
    // first); descriptor values are checked against the plan.
    static_assert(!FUSED, "partitions fold in the combine kernel");
    const int32_t* part = p.partition;
    const int h = (int)(blockIdx.x % (unsigned)p.num_kv_heads);
    const int item = (int)(blockIdx.x / (unsigned)p.num_kv_heads);
    const int L = part[1];
    if (part[2] != p.batch || L <= 0 || item >= part[0]) return;
    int x = item * L;
    const int xe = min(x + L, part[4 + p.batch]);
    for (int b = part[5 + p.batch + item]; x < xe && b >= 0 && b < p.batch; ++b) {
      const int pb = part[4 + b], pb1 = part[5 + b];
      if (pb1 <= x) continue;                     // empty request
      const int j = item - pb / L;
      if (j < 0 || j >= p.num_splits || x < pb) return;
      if (x != item * L) __syncthreads();          // the previous piece has read the shared tables
      piece(b, h, j, x - pb, min(xe, pb1) - pb);
      x = min(xe, pb1);
    }
  }
}

}  // namespace da
