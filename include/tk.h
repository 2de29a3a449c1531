/*
 * tk.h -- C ABI of libtk: counter-based random bulk fills into the device memory of one
 * AMD Instinct MI355X (gfx950).
 *
 * Contract (tandem-sycl, "Design", §Fills and §Normals): element k of a fill takes draw
 * i = start_draw + k, and its value is a pure function of (key, i).  A fill cut at any
 * element therefore equals the whole fill, and resuming a fill is a call with a larger
 * start_draw.  A start draw is an offset into the stream (tandem-cuda, "Performance",
 * §GPU: a row's start draw is a generator offset).
 *
 * Generator (Phobos stdlib, "Random numbers", §hash32 and §uniform): the lowbias32 hash,
 * word(key, c) = hash32(c ^ hash32(key)) for 32-bit key and counter.  Word c is the
 * stream's c-th 32-bit word; narrower draws are its little-endian parts and 64-bit draws
 * are the word pair (2i, 2i+1), low word first.  A fill whose counters would reach 2^32
 * is refused with TK_ERANGE instead of wrapping.
 *
 * Conventions for every call:
 *   - Pointers `out`, `x`, `y`, `mask` are device pointers owned by the caller; they must
 *     stay valid until the work enqueued on `stream` has finished.  The library never
 *     keeps them.  `out` must be aligned to its element size; any such alignment is
 *     accepted and fills at full speed (16-byte stores from the first 4 KiB boundary of
 *     `out`, the elements before it one at a time).
 *   - Calls are asynchronous and ordered on `stream` (NULL = the device's null stream)
 *     on the device current to the calling host thread.  Any host thread may call.
 *   - Arguments are checked before anything is enqueued; on any error nothing is
 *     enqueued.  n == 0 is TK_OK and enqueues nothing.  There is no CPU fallback.
 *   - TK_EHIP reports a HIP runtime failure; tk_last_hip_error() gives its code for the
 *     calling thread.
 *   - HIP graphs: a fill enqueues only kernel launches on `stream`, so it can be captured
 *     into a graph and replayed.  The first f64 normal fill on a device creates the
 *     library's per-device tables (an allocation and a copy), so run it once before
 *     capturing; alias tables are built and uploaded by tk_alias_create, outside any
 *     capture.  The test-hook modes of tk_debug_set_normal_f64_mode and the two-kernel
 *     path order fills by an event and are not meant for capture.
 */
#ifndef TK_H
#define TK_H

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum tk_status {
    TK_OK = 0,
    TK_EINVAL = 1, /* bad argument: NULL pointer, misaligned pointer, bad bound or p */
    TK_ERANGE = 2, /* draws beyond the 2^32-word counter space, or a bounded range whose
                      top does not fit the output type */
    TK_ENOMEM = 3, /* the library could not allocate its own device state */
    TK_EHIP = 4    /* a HIP runtime call failed */
} tk_status;

/* ---- Uniform fills ------------------------------------------------------------------
 * tandem-cuda, "Performance", §GPU table (fill_u8 ... fill_bool rows); narrow types write
 * fewer bytes of the same stream.
 *   u8:  draw i is byte i&3 of word i>>2          (i < 2^34)
 *   u16: draw i is half i&1 of word i>>1          (i < 2^33)
 *   u32: draw i is word i                         (i < 2^32)
 *   u64: draw i is word 2i | word 2i+1 << 32      (i < 2^31)
 *   f16_bits: binary16 encoding of (u16 draw & 0x7FF) * 2^-11, a uniform on [0, 1)
 *   f32: (word i & 0x7FFFFF) * 2^-23 (Phobos, §uniform), exactly
 *   f64: (u64 draw & (2^53 - 1)) * 2^-53, exactly
 *   bool: bit i&31 of word i>>5 as one byte 0 or 1 (tandem-sycl, "Design", §Fills: one
 *         byte per bit)                           (i < 2^37)                              */
tk_status tk_fill_u8(uint32_t key, uint64_t start_draw, uint64_t n, uint8_t *out, hipStream_t stream);
tk_status tk_fill_u16(uint32_t key, uint64_t start_draw, uint64_t n, uint16_t *out, hipStream_t stream);
tk_status tk_fill_u32(uint32_t key, uint64_t start_draw, uint64_t n, uint32_t *out, hipStream_t stream);
tk_status tk_fill_u64(uint32_t key, uint64_t start_draw, uint64_t n, uint64_t *out, hipStream_t stream);
tk_status tk_fill_f16_bits(uint32_t key, uint64_t start_draw, uint64_t n, uint16_t *out, hipStream_t stream);
tk_status tk_fill_f32(uint32_t key, uint64_t start_draw, uint64_t n, float *out, hipStream_t stream);
tk_status tk_fill_f64(uint32_t key, uint64_t start_draw, uint64_t n, double *out, hipStream_t stream);
tk_status tk_fill_bool(uint32_t key, uint64_t start_draw, uint64_t n, uint8_t *out, hipStream_t stream);

/* ---- Bounded integers ---------------------------------------------------------------
 * tandem-cuda, "Performance", §GPU (fill_u32_below, fill_u64_below, "with a low bound"
 * into int32_t / int64_t); perturbation-kernel, "Backends", §Why the GPU can be exact
 * (Lemire's multiply-shift with rejection).  Value = high half of x * bound for the
 * draw x, rejected while the low half is below (2^W - bound) mod bound; a rejected draw
 * continues on the per-index substream split(i) of sub(key, "BL32"/"BL64").
 * bound == 0 -> TK_EINVAL.  With `low`, values are low + [0, bound); a top
 * low + bound - 1 beyond the output type -> TK_ERANGE.
 *   u32_below, i32_below, i64_below32: one word per element (i < 2^32)
 *   u64_below, i64_below: one 64-bit draw per element (i < 2^31)                         */
tk_status tk_fill_u32_below(uint32_t key, uint64_t start_draw, uint64_t n, uint32_t bound,
                            uint32_t *out, hipStream_t stream);
tk_status tk_fill_u64_below(uint32_t key, uint64_t start_draw, uint64_t n, uint64_t bound,
                            uint64_t *out, hipStream_t stream);
tk_status tk_fill_i32_below(uint32_t key, uint64_t start_draw, uint64_t n, int32_t low,
                            uint32_t bound, int32_t *out, hipStream_t stream);
tk_status tk_fill_i64_below32(uint32_t key, uint64_t start_draw, uint64_t n, int64_t low,
                              uint32_t bound, int64_t *out, hipStream_t stream);
tk_status tk_fill_i64_below(uint32_t key, uint64_t start_draw, uint64_t n, int64_t low,
                            uint64_t bound, int64_t *out, hipStream_t stream);

/* ---- Normals ------------------------------------------------------------------------
 * f64 (tandem-sycl, "Design", §Normals): the 1024-layer equal-area ziggurat, one 64-bit
 * draw d per element: layer d & 1023, sign bit 10, u = (d >> 11) 2^-53; x = u X[layer] is
 * taken when below X[layer+1]; the ~0.43 % of draws that miss continue on the
 * per-index substream split(i) of sub(key, "NORM") (wedge test against exp(-x^2/2), or
 * the tail beyond r).  A table pass writes the fast-path values; the misses are finished
 * either by the same work-group after its stores or by a continuation pass over a miss
 * list (tk_debug_set_normal_f64_mode).  The 16 KiB layer table is constant per-device
 * library state; the miss lists and counts of the two-kernel path (and of counted test
 * fills) are per-device state ordered across streams by an event, while the default fused
 * fill keeps no mutable state and runs concurrently with fills on other streams.
 * i < 2^31.
 * f32 (tandem-sycl, "Design", §Normals; Phobos, §randn): Box-Muller pairs; draw i
 * belongs to pair c = i >> 1 built from the f32 uniforms at words 2c and 2c+1:
 * r = sqrt(-2 ln(1 - u1)), angle 2 pi t with t = u2 wrapped into [-1/2, 1/2); even i
 * takes r cos, odd i r sin.  i < 2^32.                                                   */
tk_status tk_fill_normal_f64(uint32_t key, uint64_t start_draw, uint64_t n, double *out, hipStream_t stream);
tk_status tk_fill_normal_f32(uint32_t key, uint64_t start_draw, uint64_t n, float *out, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, serving
 * loops, harnesses that forbid hipMalloc): tk_fill_normal_f64 computed by its two-kernel
 * path (table pass, then a continuation pass over the listed misses; the same values as
 * tk_fill_normal_f64) with no allocation of any kind.  The layer tables are compiled into
 * the library's device code, and the miss lists live in one static device array per device
 * (2.28 MiB, held from the first call on that device until the process ends); the call
 * enqueues three kernel launches on `stream` and nothing else.
 *   n: at most 2^24 elements per call, else TK_EINVAL (cut a longer fill into pieces on
 *      one stream: the pieces equal the whole fill).  Other arguments and errors as for
 *      tk_fill_normal_f64 (out 8-byte aligned, i < 2^31).
 *   Every call on a device uses that device's one array: calls that overlap in time on one
 *   device (other streams, other threads) race and give wrong values.  Order them, e.g. on
 *   one stream.  The array keeps the last call's contents; each call clears what must start
 *   at zero itself.                                                                      */
tk_status tk_fill_normal_f64_no_alloc(uint32_t key, uint64_t start_draw, uint64_t n, double *out,
                                      hipStream_t stream);

/* Normal variants (f32, i < 2^32 unless stated).
 * half_turn: tandem-sycl, "Design", §Normals shifts the Box-Muller angle by half a turn
 *   into [-pi, pi): the same pairs with angle 2 pi (u2 - 1/2), so both values are the
 *   negation of tk_fill_normal_f32's.
 * randn: Phobos, §randn, one normal per counter: element k is randn(key, start_draw + k),
 *   the cosine of Box-Muller pair start_draw + k (words 2c and 2c+1), i.e. element
 *   2 (start_draw + k) of tk_fill_normal_f32.  i < 2^31.                                 */
tk_status tk_fill_normal_f32_half_turn(uint32_t key, uint64_t start_draw, uint64_t n, float *out,
                                       hipStream_t stream);
tk_status tk_fill_randn_f32(uint32_t key, uint64_t start_draw, uint64_t n, float *out, hipStream_t stream);

/* ---- Exponentials ------------------------------------------------------------------
 * tandem-sycl, "Design", §Exponentials; tandem-cuda, "Performance", §GPU (the f32
 * exponential maps 1 - exp(-x) back to the draw's own 2^-24 grid point).  x = -ln(1 - u),
 * +0.0 at u = 0, by inversion of the draw's uniform:
 *   f64: u = (u64 draw & (2^53 - 1)) 2^-53; x from the library's table-driven f64
 *        logarithm (within 0.52 ulp of the exact value).                (i < 2^31)
 *   f32: u = (word i & 0xFFFFFF) 2^-24; x correctly rounded to f32 (the same logarithm
 *        rounded once, which is exact at every one of the 2^24 grid points).  (i < 2^32) */
tk_status tk_fill_exponential_f64(uint32_t key, uint64_t start_draw, uint64_t n, double *out, hipStream_t stream);
tk_status tk_fill_exponential_f32(uint32_t key, uint64_t start_draw, uint64_t n, float *out, hipStream_t stream);

/* ---- Fused dropout ------------------------------------------------------------------
 * Phobos, §dropout: y[k] = uniform(key, start_draw + k) >= p ? x[k] / (1 - p) : +0.0, with
 * 1 - p and the quotient rounded as f32 operations (a true division).  p must lie in
 * [0, 1), else TK_EINVAL.  x and y are n floats; they may be the same buffer (in place)
 * but must not otherwise overlap.  mask (nullable) receives one byte per element, 1 for
 * kept.  i < 2^32.                                                                       */
tk_status tk_dropout_f32(uint32_t key, uint64_t start_draw, uint64_t n, float p, const float *x,
                         float *y, uint8_t *mask, hipStream_t stream);

/* Dropout backward by redrawing (Phobos, §Random numbers: the same seed and counter give
 * the same number, so a backward pass redraws its forward pass's mask instead of storing
 * it): dx[k] = keep(k) ? dy[k] / (1 - p) : +0.0, where keep(k) is the decision of
 * tk_dropout_f32 for the same key, start_draw + k and p.  The same computation as the
 * forward call applied to dy with no mask output; same checks (dy and dx may be the same
 * buffer, no other overlap).  i < 2^32.                                                 */
tk_status tk_dropout_backward_f32(uint32_t key, uint64_t start_draw, uint64_t n, float p, const float *dy,
                                  float *dx, hipStream_t stream);

/* ---- Weighted choice through an alias table -----------------------------------------
 * tandem-sycl, "Design", §Fills: the choice fill maps each 64-bit draw through an alias
 * table.  tk_alias_create builds the table on the host from n >= 1 finite, non-negative
 * host weights with a positive sum (integer Vose construction: index j owns an integer
 * share of n * 2^32, the rounding remainder going to the largest weight) and uploads it
 * to the current device; it is synchronous and owns its device memory until
 * tk_alias_destroy.  The fill maps draw d to column c = (hi32(d) * n) >> 32 and coin
 * lo32(d): out = coin < q[c] ? c : alias[c].  The table must outlive the stream work that
 * reads it and be used on the device it was created on.  i < 2^31.                       */
typedef struct tk_alias tk_alias;
tk_status tk_alias_create(const double *weights, uint32_t n, tk_alias **table);
tk_status tk_alias_destroy(tk_alias *table);
uint32_t tk_alias_size(const tk_alias *table);
/* The host construction tk_alias_create uploads, alone: writes n entries of q and alias
 * to host arrays.  Touches no device. */
tk_status tk_alias_build_host(const double *weights, uint32_t n, uint32_t *q, uint32_t *alias);
/* Copies the table to host arrays of tk_alias_size() entries each. */
tk_status tk_alias_export(const tk_alias *table, uint32_t *q, uint32_t *alias);
tk_status tk_fill_choice_u32(uint32_t key, uint64_t start_draw, uint64_t n, const tk_alias *table,
                             uint32_t *out, hipStream_t stream);

/* ---- Philox4x32-10 word source ------------------------------------------------------
 * The counter-based generator of the cuRAND comparison column (tandem-cuda,
 * "Performance", §GPU); Salmon et al., SC'11.  64-bit key (lo, hi); word w is lane w & 3
 * of the block with counter (lo32(w >> 2), hi32(w >> 2), 0, 0).  Same draw layout and
 * float transforms as the lowbias32 fills; the counter space is 64-bit.                  */
tk_status tk_philox_fill_u32(uint64_t key, uint64_t start_draw, uint64_t n, uint32_t *out, hipStream_t stream);
tk_status tk_philox_fill_u64(uint64_t key, uint64_t start_draw, uint64_t n, uint64_t *out, hipStream_t stream);
tk_status tk_philox_fill_f32(uint64_t key, uint64_t start_draw, uint64_t n, float *out, hipStream_t stream);
tk_status tk_philox_fill_f64(uint64_t key, uint64_t start_draw, uint64_t n, double *out, hipStream_t stream);

/* Philox variants of the bounded, choice and normal fills: the same definitions as the
 * lowbias32 fills above, over Philox words (u32 draw i = word i; 64-bit draw i = words 2i
 * and 2i+1).  A draw that is rejected (Lemire) or misses the ziggurat's fast path continues
 * on its Philox substream: word j of draw i's substream for purpose P ("BL32", "BL64",
 * "NORM") is lane j & 3 of the block with counter (lo32 i, hi32 i, P, j >> 2), disjoint
 * from the primary blocks.  Limits: u32_below and normal_f32 i < 2^64, u64_below, choice
 * and normal_f64 i < 2^63; normal_f64 takes n < 2^32 per call (cut a longer fill: the
 * pieces equal the whole).  bound == 0 is TK_EINVAL.  The choice table must be on the
 * current device, as for tk_fill_choice_u32.                                            */
tk_status tk_philox_fill_u32_below(uint64_t key, uint64_t start_draw, uint64_t n, uint32_t bound, uint32_t *out,
                                   hipStream_t stream);
tk_status tk_philox_fill_u64_below(uint64_t key, uint64_t start_draw, uint64_t n, uint64_t bound, uint64_t *out,
                                   hipStream_t stream);
tk_status tk_philox_fill_choice_u32(uint64_t key, uint64_t start_draw, uint64_t n, const tk_alias *table,
                                    uint32_t *out, hipStream_t stream);
tk_status tk_philox_fill_normal_f32(uint64_t key, uint64_t start_draw, uint64_t n, float *out, hipStream_t stream);
tk_status tk_philox_fill_normal_f64(uint64_t key, uint64_t start_draw, uint64_t n, double *out, hipStream_t stream);

/* ---- Store ceiling ------------------------------------------------------------------
 * The store path alone: out[k] = value for k < n, written with exactly the streaming
 * fills' geometry, grid and 16-byte stores and no generator.  The rate at which the device
 * takes this kernel's stores is the measured ceiling the fills are reported against (the
 * pages' fills run at ~95 % of their GPU's bandwidth: tandem-cuda, "Performance", §GPU and
 * the notes under its table).  out must be 4-byte aligned; n * 4 must fit 64 bits, else
 * TK_ERANGE.                                                                            */
tk_status tk_fill_constant_u32(uint32_t value, uint64_t n, uint32_t *out, hipStream_t stream);

/* ---- Status and introspection -------------------------------------------------------*/
const char *tk_status_string(tk_status status);
/* The hipError_t of the last TK_EHIP returned to the calling thread (0 if none). */
int tk_last_hip_error(void);
/* Copies the 1024-layer table the kernels use: x and f of 1025 doubles each (host). */
tk_status tk_ziggurat_table(double *x, double *f);
/* Test hook for the f64 normal's miss lists, applied from the next tk_fill_normal_f64 on
 * every device: each table-pass work-group keeps at most `per_group` misses (1..16) in its
 * queue.  In the two-kernel mode the rest go to an overflow list of `overflow` entries,
 * and when that overflows too the continuation pass walks the whole fill; in the fused
 * mode a group with more misses walks its own elements again.  0 restores the defaults
 * (16 per 4 KiB tile, 65536 overflow entries).  Lets tests force every fallback. */
tk_status tk_debug_set_miss_capacity(uint32_t per_group, uint64_t overflow);
/* Test hook: how tk_fill_normal_f64 finishes its misses, from the next call on every
 * device: 1 = the two-kernel path (table pass, then a continuation pass over the listed
 * misses), 2 = fused (each table-pass work-group finishes its own misses after its
 * stores), 0 = the library default.  Both give identical results. */
tk_status tk_debug_set_normal_f64_mode(uint32_t mode);
/* Test hook: waits for the current device's last tk_fill_normal_f64 and returns how many
 * of its draws missed the fast path (synchronous).  The counts are kept only while a mode
 * is chosen with tk_debug_set_normal_f64_mode (1 or 2), or when the library default is
 * the two-kernel path; after a fill in the default fused mode, which keeps no per-device
 * state and is not ordered against fills on other streams, it returns TK_EINVAL. */
tk_status tk_debug_last_miss_count(uint64_t *count);
/* Test hook: of the library's next device allocations (a device's ziggurat tables on its
 * first f64 normal fill, the two-kernel path's miss lists as they grow, alias tables), the
 * first `skip` proceed and the `count` after them fail as if device memory were exhausted,
 * without calling HIP.  The call that needed the memory returns TK_ENOMEM, enqueues
 * nothing and holds no more device memory than before it (a first fill releases the
 * tables it created; a failed growth releases all the miss lists); a later call allocates
 * again.  count = 0 cancels.  Process-wide, for every device and thread.  A real
 * allocation failure takes the same path.  The environment variable TK_DEBUG_FAIL_ALLOC=<n>
 * makes the process's first n allocations fail the same way (a call here replaces it), and
 * the library says so once on stderr. */
tk_status tk_debug_fail_allocations(uint32_t skip, uint32_t count);
/* Test hook: the device memory the library holds now, in bytes, over all devices: the
 * per-device ziggurat state (held until the process ends) and the live alias tables. */
tk_status tk_debug_device_bytes(uint64_t *bytes);
/* Test and benchmark hook: sets a launch tunable for every later call in the process (the
 * defaults, read from TK_* environment variables at first use, are the measured best).
 * Results never depend on them; they choose among launch shapes that compute the same
 * values.  `name` and the accepted values:
 *   "store_nt" 0|1        non-temporal 16-byte stores in the streaming fills (TK_STORE=nt)
 *   "max_blocks" 1..2^31-1  grid cap of the streaming fills, which then stride (TK_MAX_BLOCKS)
 *   "unroll" 1|2|4        16-byte vectors per lane per tile in the streaming fills (TK_UNROLL)
 *   "choice_tiles" 1|2|4|8  4 KiB tiles per choice work-group (TK_CHOICE_TILES)
 *   "exp_tiles" 1|2|4     tiles per exponential work-group (TK_EXP_TILES)
 *   "zig_tiles" 1|2|4|8|16  tiles per ziggurat table-pass work-group (TK_ZIG_TILES)
 *   "zig_lds" 0|1         ziggurat layer gathers from an LDS copy or from L1/L2 (TK_ZIG_TABLE)
 *   "zig_fused" 0|1       ziggurat misses finished in the table pass or a second kernel
 *                         (TK_ZIG_MODE; tk_debug_set_normal_f64_mode overrides it)
 *   "philox_lds" 0|1      Philox fills at word offsets 1..3 by the LDS tile kernel (1) or
 *                         the overlapping-wave kernel (0) (TK_PHILOX=lds|overlap)
 *   "pair_lds" 0|1        lowbias32 Box-Muller fills at odd starts by the pair tile kernel,
 *                         which passes each wave's first value on through LDS (1), or with
 *                         every wave computing the value after it itself (0)
 *                         (TK_PAIRS=lds|wave)
 *   "lds_pad" 0..65536    dynamic LDS bytes allocated per work-group of every fill but the
 *                         ziggurat (for choice, on top of its table), which caps the groups a
 *                         compute unit holds at once (TK_LDS_PAD; unset: each fill's measured
 *                         default, 24 or 32 KiB for the integer fills, else none)
 *   "zig_lds_pad" 0..65536  the same for the ziggurat table pass (TK_ZIG_LDS_PAD)
 *   "const_work" 0..4096  dependent integer steps per lane before each store of
 *                         tk_fill_constant_u32 (TK_CONST_WORK; 0 = none): the spacing of
 *                         the store-ceiling measurement
 * A negative value restores the environment's setting.  Unknown names or values: TK_EINVAL.
 * Not synchronized with launches in flight on other threads beyond each value being read
 * atomically. */
tk_status tk_debug_set_tunable(const char *name, int64_t value);

#ifdef __cplusplus
}
#endif
#endif
