/*
 * oracle.c -- plain, slow CPU reference for the float8 MoE quantization path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or calls
 * this file; only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark do.  It shares no code, header, table or constant with the HIP
 * library: every value below is computed from the definitions, in double
 * precision where the arithmetic is exact and in IEEE binary32 exactly where the
 * group-scaling definition fixes binary32 (its scales are fp32).
 *
 * Sources (the pages this follows):
 *   [A2A]  "[mxfp8 MoE training] Support mxfp8 all to all in expert parallel"
 *          (torchtitan PR 1765), Summary: the payload is quantized to mxfp8,
 *          e4m3 data and e8m0 scales are exchanged, and the receiver turns them
 *          back into bf16, the input's precision.
 *   [GRP]  "[moe training] fix uncoalesced global accesses in per group rowwise
 *          scaling kernel" (torchao PR 2761), Summary: per-group float8 scaling
 *          whose output feeds the LHS of a scaled grouped GEMM, written row-major
 *          or column-major (then transformed).  The grouped product itself
 *          (token rows of group g times the transpose of expert g's weight, both
 *          as MXFP8) is the MoE GEMM configuration built on these operands.
 *   MXFP8 itself is the OCP Microscaling (MX) v1.0 format that the name refers
 *   to: blocks of 32 elements share one E8M0 power-of-two scale whose exponent
 *   is floor(log2(amax)) minus the element format's largest exponent (8 for
 *   E4M3); elements are E4M3 (OCP "fn" variant: bias 7, max 448, NaN = S.1111.111).
 *
 * Readings where the pages are silent (all are also listed with the design
 * notes of the repository):
 *   - block of 32 contiguous elements along the last dimension;
 *   - round-to-nearest, ties to even, saturating to +-448; signs kept (-0 stays);
 *   - scale exponent clamped to [-127, 127]; an all-zero or subnormal block
 *     gets code 0; a block holding Inf or NaN gets scale 0xFF and payload 0x7F;
 *   - dequantized values are rounded once (RNE) to bf16, subnormals kept,
 *     NaN written as 0x7FC0;
 *   - group scaling: s = 448 / max(amax, 1e-12) in fp32, q = e4m3(fp32(x*s)),
 *     the fp32 multiplier s is the stored scale; a column with Inf/NaN gets
 *     s = NaN and payload 0x7F; group g spans rows [end(g-1), end(g)) with the
 *     end offsets clamped to be non-decreasing and <= M; rows past the last end
 *     get 0x00;
 *   - grouped product: operands are MXFP8 along K (the contraction dimension);
 *     the reference value is the double-precision sum of the exactly
 *     dequantized products; rows past the last end give 0.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fPIC -shared
 * (x86-64 SSE arithmetic: binary32 ops are correctly rounded, no x87 excess
 * precision).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define ORACLE_ABI 1

int oracle_abi_version(void) { return ORACLE_ABI; }

/* ---------------------------------------------------------------- bf16 ---- */

/* Value of a bf16 bit pattern (the upper half of a binary32). */
double oracle_bf16_value(uint16_t bits)
{
    uint32_t w = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

static int is_finite_d(double v) { return !isnan(v) && !isinf(v); }

/* floor(log2(a)) for finite a > 0, exact (frexp returns a = f * 2^e, f in [0.5, 1)). */
static int floor_log2(double a)
{
    int e;
    (void)frexp(a, &e);
    return e - 1;
}

/* Round a finite or infinite double once to bf16 (8 significant bits, exponent
 * range of binary32), ties to even, subnormals kept, overflow to Inf.
 * NaN becomes the canonical 0x7FC0. */
uint16_t oracle_bf16_round(double v)
{
    if (isnan(v)) return 0x7FC0;
    uint16_t sign = signbit(v) ? 0x8000 : 0x0000;
    double a = fabs(v);
    if (isinf(a)) return sign | 0x7F80;
    if (a == 0.0) return sign;
    int ex = floor_log2(a);
    if (ex < -126) ex = -126;                 /* subnormal binade shares 2^-133 spacing */
    double quantum = ldexp(1.0, ex - 7);      /* 7 stored mantissa bits */
    double r = rint(a / quantum) * quantum;   /* a/quantum is exact; rint = ties-to-even */
    if (r >= ldexp(1.0, 128)) return sign | 0x7F80;
    if (r < ldexp(1.0, -126)) {               /* subnormal: r = m * 2^-133 */
        return sign | (uint16_t)(r / ldexp(1.0, -133));
    }
    int e = floor_log2(r);
    uint16_t mant = (uint16_t)((r / ldexp(1.0, e) - 1.0) * 128.0);
    return sign | (uint16_t)((e + 127) << 7) | mant;
}

/* ---------------------------------------------------------------- e4m3 ---- */

/* Decode an OCP E4M3 ("fn") code: S.EEEE.MMM, bias 7; E=0 is subnormal
 * (m/8 * 2^-6); S.1111.111 is NaN; there is no infinity. */
double oracle_e4m3_decode(uint8_t code)
{
    int s = code >> 7, E = (code >> 3) & 0xF, m = code & 0x7;
    if (E == 15 && m == 7) return NAN;
    double mag = (E == 0) ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, E - 7);
    return s ? -mag : mag;
}

/* Nearest E4M3 magnitude to a >= 0 (finite), ties to even, saturated to 448. */
static double e4m3_round_magnitude(double a)
{
    if (a == 0.0) return 0.0;
    int ex = floor_log2(a);
    if (ex < -6) ex = -6;                     /* subnormals share the 2^-9 spacing */
    double quantum = ldexp(1.0, ex - 3);      /* 3 stored mantissa bits */
    double r = rint(a / quantum) * quantum;
    if (r > 448.0) r = 448.0;                 /* saturate (480 and up are not E4M3 values) */
    return r;
}

/* Bit pattern of an exact, non-negative E4M3 magnitude. */
static uint8_t e4m3_magnitude_bits(double r)
{
    if (r == 0.0) return 0;
    if (r < ldexp(1.0, -6)) return (uint8_t)(r / ldexp(1.0, -9));  /* subnormal: m * 2^-9 */
    int e = floor_log2(r);
    uint8_t mant = (uint8_t)((r / ldexp(1.0, e) - 1.0) * 8.0);
    return (uint8_t)(((e + 7) << 3) | mant);
}

/* Encode a finite double to E4M3: round to nearest, ties to even, saturate to
 * +-448, sign copied (so -0 and small negatives give 0x80). */
uint8_t oracle_e4m3_encode(double y)
{
    uint8_t sign = signbit(y) ? 0x80 : 0x00;
    if (isnan(y)) return 0x7F;
    double a = fabs(y);
    if (isinf(a)) return sign | 0x7E;         /* saturating */
    return sign | e4m3_magnitude_bits(e4m3_round_magnitude(a));
}

/* ---------------------------------------------------------------- e8m0 ---- */

/* E8M0 scale: 2^(c - 127); 0xFF is NaN. */
double oracle_e8m0_decode(uint8_t code)
{
    if (code == 0xFF) return NAN;
    return ldexp(1.0, (int)code - 127);
}

/* ------------------------------------------------------------- MXFP8 ------ */

/* Shared exponent of one block of n values: floor(log2(amax)) - 8, clamped to
 * [-127, 127] (amax = 0 counts as -infinity and clamps to -127).  Returns the
 * E8M0 code, or 0xFF if the block holds Inf or NaN. */
static uint8_t mx_block_scale_code(const double* v, int n)
{
    double amax = 0.0;
    for (int i = 0; i < n; ++i) {
        if (!is_finite_d(v[i])) return 0xFF;
        double a = fabs(v[i]);
        if (a > amax) amax = a;
    }
    int shared = (amax == 0.0) ? -127 : floor_log2(amax) - 8;
    if (shared < -127) shared = -127;
    if (shared > 127) shared = 127;
    return (uint8_t)(shared + 127);
}

/* MX quantize one element given its block's scale code (finite block). */
uint8_t oracle_mx_encode_element(uint16_t xbits, uint8_t scale_code)
{
    double x = oracle_bf16_value(xbits);
    double y = x / ldexp(1.0, (int)scale_code - 127);  /* exact: power-of-two divide */
    return oracle_e4m3_encode(y);
}

/* X: (M, K) bf16 bits, row-major, K % 32 == 0.
 * Q: (M, K) E4M3 codes, row-major.  S: (M, K/32) E8M0 codes, row-major. */
void oracle_mx_quantize(const uint16_t* x, int64_t M, int64_t K, uint8_t* q, uint8_t* s)
{
    const int64_t nb = K / 32;
    double v[32];
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t b = 0; b < nb; ++b) {
            const uint16_t* xb = x + m * K + b * 32;
            for (int i = 0; i < 32; ++i) v[i] = oracle_bf16_value(xb[i]);
            uint8_t c = mx_block_scale_code(v, 32);
            s[m * nb + b] = c;
            uint8_t* qb = q + m * K + b * 32;
            if (c == 0xFF) {
                for (int i = 0; i < 32; ++i) qb[i] = 0x7F;
                continue;
            }
            double scale = oracle_e8m0_decode(c);
            for (int i = 0; i < 32; ++i) qb[i] = oracle_e4m3_encode(v[i] / scale);
        }
    }
}

/* Dequantize one element: round_bf16(e4m3(q) * 2^(c-127)); NaN code or NaN
 * scale gives 0x7FC0. */
uint16_t oracle_mx_decode_element(uint8_t q, uint8_t scale_code)
{
    double d = oracle_e4m3_decode(q);
    double sc = oracle_e8m0_decode(scale_code);
    if (isnan(d) || isnan(sc)) return 0x7FC0;
    return oracle_bf16_round(d * sc);         /* product is exact in double */
}

void oracle_mx_dequantize(const uint8_t* q, const uint8_t* s, int64_t M, int64_t K, uint16_t* y)
{
    const int64_t nb = K / 32;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k)
            y[m * K + k] = oracle_mx_decode_element(q[m * K + k], s[m * nb + k / 32]);
}

/* ------------------------------------------------- MX variants ------------ */
/* Two variants of the MX quantizer that the MX v1.0 definition above leaves to
 * the user of the format, both readings of this repository (the pages name
 * mxfp8 only):
 *   scale rule RCEIL: the shared exponent is the smallest integer e for which
 *     amax <= 448 * 2^e, i.e. ceil(log2(amax / 448)): the scale is rounded up
 *     so that no element of the block exceeds 448 once scaled and nothing
 *     saturates.  Clamped to [-127, 127] like the floor rule; amax = 0 gives
 *     -127.
 *   axis 0: blocks of 32 consecutive rows of one column (the layout a GEMM that
 *     contracts over tokens needs), instead of 32 consecutive elements of a row.
 * rule: 0 = floor (the rule above), 1 = RCEIL.  axis: 1 = along rows (K), 0 =
 * along columns (M). */
static int mx_shared_exponent(double amax, int rule)
{
    int e;
    if (amax == 0.0) {
        e = -127;
    } else if (rule == 0) {
        e = -8 + floor_log2(amax);             /* the floor rule, as mx_block_scale_code */
    } else {
        e = floor_log2(amax) - 9;              /* 448 * 2^e = 0.875 * 2^floor_log2 < amax */
        while (amax > 448.0 * ldexp(1.0, e)) ++e;
    }
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e;
}

/* Index of element i (0..31) of block (a, b): axis 1 -> row a, columns 32b..;
 * axis 0 -> rows 32a.., column b. */
static int64_t mx_block_index(int axis, int64_t K, int64_t a, int64_t b, int i)
{
    return axis == 1 ? a * K + b * 32 + i : (a * 32 + i) * K + b;
}

/* X: (M, K) bf16 bits row-major; Q: (M, K) E4M3 in the same layout as X.
 * axis 1: K % 32 == 0, S (M, K/32) row-major, S[m][b] for columns 32b..32b+31.
 * axis 0: M % 32 == 0, S (M/32, K) row-major, S[a][k] for rows 32a..32a+31. */
void oracle_mx_quantize_ex(const uint16_t* x, int64_t M, int64_t K, int axis, int rule, uint8_t* q, uint8_t* s)
{
    const int64_t na = axis == 1 ? M : M / 32;     /* blocks: na x nb */
    const int64_t nb = axis == 1 ? K / 32 : K;
    double v[32];
    for (int64_t a = 0; a < na; ++a) {
        for (int64_t b = 0; b < nb; ++b) {
            double amax = 0.0;
            int finite = 1;
            for (int i = 0; i < 32; ++i) {
                v[i] = oracle_bf16_value(x[mx_block_index(axis, K, a, b, i)]);
                if (!is_finite_d(v[i])) finite = 0;
                else if (fabs(v[i]) > amax) amax = fabs(v[i]);
            }
            if (!finite) {
                s[a * nb + b] = 0xFF;
                for (int i = 0; i < 32; ++i) q[mx_block_index(axis, K, a, b, i)] = 0x7F;
                continue;
            }
            const int e = mx_shared_exponent(amax, rule);
            s[a * nb + b] = (uint8_t)(e + 127);
            for (int i = 0; i < 32; ++i)
                q[mx_block_index(axis, K, a, b, i)] = oracle_e4m3_encode(v[i] / ldexp(1.0, e));
        }
    }
}

/* Inverse of oracle_mx_quantize_ex for either axis: each element is decoded
 * with its own block's scale exactly as oracle_mx_decode_element does. */
void oracle_mx_dequantize_ex(const uint8_t* q, const uint8_t* s, int64_t M, int64_t K, int axis, uint16_t* y)
{
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k) {
            const uint8_t c = axis == 1 ? s[m * (K / 32) + k / 32] : s[(m / 32) * K + k];
            y[m * K + k] = oracle_mx_decode_element(q[m * K + k], c);
        }
}

/* ------------------------------------------------------ group scaling ----- */

/* binary32 helpers: every operation here is one correctly rounded IEEE op. */
static float f32_of_bf16(uint16_t bits)
{
    uint32_t w = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return f;
}

/* Scale of one (group, column): s = 448 / max(amax, 1e-12) in binary32. */
float oracle_group_scale_value(float amax)
{
    volatile float denom = amax > 1e-12f ? amax : 1e-12f;
    volatile float s = 448.0f / denom;
    return s;
}

/* Quantize one element of a group column with multiplier s (finite):
 * the binary32 product is rounded first, then encoded to E4M3. */
uint8_t oracle_group_encode_element(uint16_t xbits, float s)
{
    volatile float p = f32_of_bf16(xbits) * s;
    return oracle_e4m3_encode((double)p);
}

/* X: (M, K) bf16 bits row-major.  group_end: G cumulative end offsets.
 * layout 0: Q[m*K + k] (same layout as X); layout 1: Q[k*M + m].
 * scales: (G, K) binary32, the multiplier applied before the cast. */
void oracle_group_scale(const uint16_t* x, int64_t M, int64_t K,
                        const int32_t* group_end, int32_t G, int layout,
                        uint8_t* q, float* scales)
{
    int64_t start = 0;
    for (int32_t g = 0; g < G; ++g) {
        int64_t end = group_end[g];
        if (end < start) end = start;
        if (end > M) end = M;
        for (int64_t k = 0; k < K; ++k) {
            double amax = 0.0;
            int finite = 1;
            for (int64_t r = start; r < end; ++r) {
                double v = oracle_bf16_value(x[r * K + k]);
                if (!is_finite_d(v)) finite = 0;
                else if (fabs(v) > amax) amax = fabs(v);
            }
            float s;
            if (!finite) {
                uint32_t nanbits = 0x7FC00000u;
                memcpy(&s, &nanbits, sizeof s);
            } else {
                s = oracle_group_scale_value((float)amax);   /* amax is a bf16 value: exact */
            }
            scales[(int64_t)g * K + k] = s;
            for (int64_t r = start; r < end; ++r) {
                uint8_t c = finite ? oracle_group_encode_element(x[r * K + k], s) : 0x7F;
                if (layout == 0) q[r * K + k] = c;
                else q[k * M + r] = c;
            }
        }
        start = end;
    }
    /* rows outside every group */
    for (int64_t r = start; r < M; ++r)
        for (int64_t k = 0; k < K; ++k) {
            if (layout == 0) q[r * K + k] = 0;
            else q[k * M + r] = 0;
        }
}

/* Group-scaling variants (readings of this repository; the pages fix neither):
 *   flag 1, power-of-two scales: the multiplier s is rounded down to a power of
 *     two, s' = 2^floor(log2 s), so that amax * s' <= 448 still holds and the
 *     scaled product x * s' is exact; q = e4m3(binary32(x * s')).
 *   flag 2, inverse scales: the stored scale is the dequantization factor
 *     1 / s (one binary32 division) instead of the multiplier; the codes are
 *     those of the multiplier convention.
 * Both flags may be combined; NaN columns store NaN either way. */
static float group_pow2_floor(float s)
{
    int e;
    (void)frexpf(s, &e);                       /* s = f * 2^e, f in [0.5, 1) */
    return ldexpf(1.0f, e - 1);
}

void oracle_group_scale_ex(const uint16_t* x, int64_t M, int64_t K,
                           const int32_t* group_end, int32_t G, int layout, int flags,
                           uint8_t* q, float* scales)
{
    int64_t start = 0;
    for (int32_t g = 0; g < G; ++g) {
        int64_t end = group_end[g];
        if (end < start) {
            end = start;                       /* running maximum of the ends */
        }
        if (end > M) end = M;
        for (int64_t k = 0; k < K; ++k) {
            double amax = 0.0;
            int finite = 1;
            for (int64_t r = start; r < end; ++r) {
                double v = oracle_bf16_value(x[r * K + k]);
                if (!is_finite_d(v)) finite = 0;
                else if (fabs(v) > amax) amax = fabs(v);
            }
            float mult, stored;
            if (!finite) {
                uint32_t nanbits = 0x7FC00000u;
                memcpy(&mult, &nanbits, sizeof mult);
                stored = mult;
            } else {
                mult = oracle_group_scale_value((float)amax);
                if (flags & 1) mult = group_pow2_floor(mult);
                volatile float one = 1.0f;
                stored = (flags & 2) ? one / mult : mult;
            }
            scales[(int64_t)g * K + k] = stored;
            for (int64_t r = start; r < end; ++r) {
                uint8_t c = finite ? oracle_group_encode_element(x[r * K + k], mult) : 0x7F;
                if (layout == 0) q[r * K + k] = c;
                else q[r + k * M] = c;
            }
        }
        start = end;                           /* the next group starts here */
    }
    for (int64_t r = start; r < M; ++r)
        for (int64_t k = 0; k < K; ++k) {
            if (layout == 0) q[r * K + k] = 0;
            else q[r + k * M] = 0;
        }
}

/* ------------------------------------------------------- dispatch pack --- */
/* [A2A] Summary: the payload of the expert-parallel all-to-all is quantized to
 * MXFP8 and sent as e4m3 data plus e8m0 scales.  The dispatch pack builds that
 * payload in one step (a reading of this repository, the pages show the two
 * buffers only): token t with expert ids[t*topk + j] (j < topk) contributes one
 * row per (t, j) pair, the pairs are ordered by expert, stably (by pair index
 * p = t*topk + j within an expert), and each row is the token's MX encoding
 * packed as [K e4m3 codes | K/32 e8m0 scales] (row stride K + K/32 bytes), so
 * that one buffer carries both parts of every row.  Pairs whose expert id is
 * outside [0, E) are dropped.  src_pair[r] is the pair index of row r;
 * group_end[e] is the number of kept pairs with expert <= e.  Rows at or past
 * group_end[E-1] are not written (their src_pair is -1). */
void oracle_dispatch_pack(const uint16_t* x, int64_t M, int64_t K, const int32_t* ids, int32_t topk,
                          int32_t E, uint8_t* packed, int32_t* src_pair, int32_t* group_end)
{
    const int64_t P = M * topk, ldp = K + K / 32;
    int64_t r = 0;
    for (int32_t e = 0; e < E; ++e) {
        for (int64_t p = 0; p < P; ++p) {
            if (ids[p] != e) continue;
            uint8_t* row = packed + r * ldp;
            oracle_mx_quantize(x + (p / topk) * K, 1, K, row, row + K);
            src_pair[r] = (int32_t)p;
            ++r;
        }
        group_end[e] = (int32_t)r;
    }
    for (; r < P; ++r) src_pair[r] = -1;
}

/* ------------------------------------------------------------ transpose --- */

/* out (C, R) = transpose of in (R, C), bytes. */
void oracle_transpose_u8(const uint8_t* in, int64_t R, int64_t C, uint8_t* out)
{
    for (int64_t i = 0; i < R; ++i)
        for (int64_t j = 0; j < C; ++j)
            out[j * R + i] = in[i * C + j];
}

/* ----------------------------------------------- scaled grouped GEMM --- */

/* Grouped product of MXFP8 operands, in double.
 * [GRP] Summary (the group-scaled tokens are the LHS of a scaled grouped GEMM)
 * and the MoE configuration "Y_g = X_g W_g^T": token rows of group g are
 * multiplied by the transpose of expert g's weight.
 *   xq (M, K) E4M3 and xs (M, K/32) E8M0: the tokens, MX blocks along K.
 *   wq (G, N, K) E4M3 and ws (G, N, K/32) E8M0: one (N, K) weight per group.
 *   group_end: G cumulative ends, clamped as in oracle_group_scale.
 * Computes y[i, j] = Y[rows[i], cols[j]] for the requested rows and columns:
 * the sum over k of x(r, k) * w_g(n, k), where each operand value is its E4M3
 * code times its block's E8M0 scale (exact in double, as is every product),
 * accumulated in double in k order.  A row at or past the last end belongs to
 * no group and gives 0.  The two 256-entry tables below only cache
 * oracle_e4m3_decode / oracle_e8m0_decode. */
void oracle_mx_grouped_mm(const uint8_t* xq, const uint8_t* xs,
                          const uint8_t* wq, const uint8_t* ws,
                          const int32_t* group_end, int64_t M, int64_t N, int64_t K,
                          int32_t G, const int64_t* rows, int64_t nrows,
                          const int64_t* cols, int64_t ncols, double* y)
{
    double e4m3[256], e8m0[256];
    for (int c = 0; c < 256; ++c) {
        e4m3[c] = oracle_e4m3_decode((uint8_t)c);
        e8m0[c] = oracle_e8m0_decode((uint8_t)c);
    }
    const int64_t KB = K / 32;
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t r = rows[i];
        /* group of row r under the clamped ends */
        int32_t grp = -1;
        int64_t start = 0;
        for (int32_t g = 0; g < G; ++g) {
            int64_t end = group_end[g];
            end = end < start ? start : end;     /* running maximum */
            end = end > M ? M : end;
            if (r >= start && r < end) { grp = g; break; }
            start = end;
        }
        for (int64_t j = 0; j < ncols; ++j) {
            int64_t n = cols[j];
            double acc = 0.0;
            if (grp >= 0) {
                const uint8_t* wrow = wq + ((int64_t)grp * N + n) * K;
                const uint8_t* wsrow = ws + ((int64_t)grp * N + n) * KB;
                const uint8_t* xrow = xq + r * K;
                const uint8_t* xsrow = xs + r * KB;
                for (int64_t k = 0; k < K; ++k) {
                    double xv = e4m3[xrow[k]] * e8m0[xsrow[k / 32]];
                    double wv = e4m3[wrow[k]] * e8m0[wsrow[k / 32]];
                    acc += xv * wv;
                }
            }
            y[i * ncols + j] = acc;
        }
    }
}

/* ------------------------------------------- element-wise array forms ----- */
/* Same functions as above, applied element by element over arrays (so that
 * exhaustive checks need not cross the FFI once per element). */

void oracle_mx_encode_elements(const uint16_t* x, const uint8_t* scale_code, int64_t n, uint8_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_mx_encode_element(x[i], scale_code[i]);
}

void oracle_mx_decode_elements(const uint8_t* q, const uint8_t* scale_code, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_mx_decode_element(q[i], scale_code[i]);
}

void oracle_e4m3_encode_f32_array(const float* y, int64_t n, uint8_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_encode((double)y[i]);
}

void oracle_bf16_round_f64_array(const double* v, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_round(v[i]);
}

void oracle_group_encode_elements(const uint16_t* x, const float* s, int64_t n, uint8_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_group_encode_element(x[i], s[i]);
}
