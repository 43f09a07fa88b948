/*
 * mxgemm.h -- C ABI of the MI355X (gfx950) low-batch MXFP8 publishing GEMM and
 * its three-generation Lamport mailbox.
 *
 * Page citations name the four API pages by module:
 *   "all_gather page"      vllm.models.deepseek_v41.nvidia.ops.cute_dsl.all_gather
 *   "publishing_gemm page" vllm.models.deepseek_v41.nvidia.specialized_decode.
 *                          boundary.publishing_gemm
 *   "sync page"            vllm.models.deepseek_v41.amd.mono.common.sync
 *
 * Conventions for every entry point:
 *   - Pointers named as device pointers are HIP device memory owned by the
 *     caller; the library never allocates, frees or keeps them.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). All
 *     work is enqueued on it; no entry point synchronizes the host, so every
 *     call except mailbox_init and mxgemm_workspace_init may be captured into
 *     a HIP graph.
 *   - Arguments are validated on the host from sizes and addresses alone
 *     (all_gather page, LamportAllGather.accepts: decided from the size, so
 *     every caller decides alike). On any error nothing is enqueued and a
 *     negative MXG_E* code is returned; 0 means enqueued.
 *   - Calls on one mailbox go on one stream, in order, and never overlap
 *     (all_gather page, module docstring, closing paragraph).
 */
#ifndef MXGEMM_H
#define MXGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- return codes ------------------------------------------------------ */
#define MXG_OK 0
#define MXG_EINVAL (-1)       /* null pointer, bad shape or rank, bad split_k */
#define MXG_EALIGN (-2)       /* a pointer is not 16-byte aligned */
#define MXG_ECAPACITY (-3)    /* payload does not fit a rank slot */
#define MXG_EWORKSPACE (-4)   /* split-K workspace missing or too small */
#define MXG_EUNSUPPORTED (-5) /* valid, but no kernel variant takes it: fall back */
#define MXG_EHIP (-6)         /* a HIP call failed (no device, launch error) */

/* ---- mailbox geometry (all_gather page, module docstring) --------------- */
#define MXG_GENERATIONS 3     /* three generations */
#define MXG_PACK_BYTES 16     /* handled in 16-byte packs */
#define MXG_SENTINEL 0x80000000u /* idle word: FP32 -0 / INT32_MIN */
#define MXG_MAX_RANKS 8
#define MXG_MAX_ROWS 8        /* at most 8 activation rows (publishing_gemm page) */
#define MXG_SCALE_BLOCK 32    /* one E8M0 scale per 32 K (sf_vec_size=32) */

/* Mailbox state words (uint32). NEXT and ACTIVE are the stage words of the
 * publishing_gemm page's module docstring: [0] the generation the owner's
 * next publish writes (advanced by the collect that empties it), [1] the
 * generation the owner's last publish wrote, which the collect reads.
 * COLLECT_ARR counts the fused all-gather's workgroups (all_gather page, step
 * 3: the last to arrive advances the generation). ERROR is a sticky bit set:
 * MXG_ERR_* below.
 *
 * PEER_GEN + r is the generation counter of emulated peer slot r (r other
 * than the owner's rank): every rank keeps its own counter and advances it
 * once per call (all_gather page, module docstring, step 3), so a peer never
 * reads the owner's NEXT, which the owner's collect advances while peers may
 * still be about to publish. A peer publish writes generation PEER_GEN[r] and
 * the last of its workgroups to arrive (PEER_ARR + r counts them) advances
 * PEER_GEN[r] mod 3. With one publish per peer per collect, PEER_GEN[r]
 * equals NEXT whenever no call is in flight. */
#define MXG_STATE_WORDS 32
#define MXG_STATE_NEXT 0
#define MXG_STATE_ACTIVE 1
#define MXG_STATE_COLLECT_ARR 2
#define MXG_STATE_ERROR 3
#define MXG_STATE_PEER_GEN 8
#define MXG_STATE_PEER_ARR 16

/* Split-K workspace layout:
 *   [0, 256)             header, uint32 words: EPOCH, (reserved), ERROR
 *   [256, 256 + 8192)    one uint32 per workgroup: the epoch it read
 *   [256 + 8192, ...)    (value, tag) pairs, see mxgemm_workspace_bytes
 * EPOCH tags every (value, tag) pair a GEMM call exchanges between its
 * workgroups (sync page, Mailbox docstring: a launch tags its hand-offs with
 * its epoch, so a pair from an earlier call never carries a live tag). Each
 * workgroup stores the epoch it read into its own word; once workgroup 0
 * has seen every word of the launch hold the epoch, it stores the next one
 * (skipping 0), so the next call, and no workgroup of this one, reads it. A
 * split-K launch has at most MXG_WS_MAX_GROUPS workgroups. */
#define MXG_WS_HEADER_BYTES 256
#define MXG_WS_FLAG_BYTES 8192
#define MXG_WS_MAX_GROUPS 2048
#define MXG_WS_EPOCH 0
#define MXG_WS_ERROR 2

#define MXG_ERR_COLLECT_SPIN 0x1u /* a collect gave up polling a slot */
#define MXG_ERR_SPLITK_SPIN 0x2u  /* a split-K owner gave up polling its pairs */

/* Default poll limit of the device waits (MXG_DEFAULT_SPIN_LIMIT polls, with
 * s_sleep between polls). */
#define MXG_DEFAULT_SPIN_LIMIT (1u << 20)

/* Host-side descriptor of one mailbox (plain data, copied freely). */
typedef struct mxg_mailbox {
  void* slots;             /* device: 3 * ranks * capacity_bytes, 16-B aligned */
  uint32_t* state;         /* device: MXG_STATE_WORDS words, 16-B aligned */
  int32_t ranks;           /* emulated rank slots, 1..8 */
  int32_t rank;            /* the slot mxgemm_publish writes, 0..ranks-1 */
  int64_t capacity_bytes;  /* bytes per rank slot, > 0, multiple of 16 */
  uint32_t spin_limit;     /* polls before a device wait of a call on this
                              mailbox gives up (its collect, its split-K
                              exchange); 0: MXG_DEFAULT_SPIN_LIMIT. mailbox_init
                              sets 0; tests set it small to force a time-out */
  uint32_t reserved;       /* 0 */
} mxg_mailbox;

/* Bytes of slot memory a mailbox needs: 3 * ranks * capacity_bytes, or 0 if
 * the arguments are invalid. */
size_t mxg_mailbox_slots_bytes(int32_t ranks, int64_t capacity_bytes);

/* Fill `mb` and arm the mailbox: every slot word becomes the sentinel and
 * every state word 0 (NEXT, ACTIVE, COLLECT_ARR, ERROR and the peer
 * counters; all_gather page, LamportAllGather.__init__: the mailbox starts as
 * the sentinel with a zero state). Enqueues fill kernels on `stream`; call it at a quiescent point,
 * outside graph capture. Errors: MXG_EINVAL (null, ranks outside 1..8, rank
 * outside 0..ranks-1, capacity not a positive multiple of 16), MXG_EALIGN,
 * MXG_EHIP. */
int mailbox_init(mxg_mailbox* mb, void* slots, uint32_t* state, int32_t ranks,
                 int32_t rank, int64_t capacity_bytes, void* stream);

/* Bytes of split-K workspace mxgemm_publish needs for these sizes: 0 when
 * split_k == 1, else MXG_WS_HEADER_BYTES + MXG_WS_FLAG_BYTES
 * + split_k * 64 * ceil(n/8)*8: eight (value, tag) pairs of 8 bytes for each
 * of 8 token rows and n/8 packs. */
size_t mxgemm_workspace_bytes(int32_t m, int32_t n, int32_t k, int32_t split_k);

/* Arm a workspace: zero every word, then EPOCH = 1. Call it
 * once before first use, outside capture; a workspace may then serve calls
 * of any size up to its capacity, in any order. Errors: MXG_EINVAL,
 * MXG_EALIGN, MXG_EHIP. */
int mxgemm_workspace_init(void* workspace, size_t workspace_bytes, void* stream);

/* Packed weight layout. The GEMM streams W as 2048-byte tiles, one per
 * (16-row block rb, 128-wide K block kb), in the order its lanes load them,
 * so that every wave instruction reads 1 KB of contiguous HBM:
 *   w_packed  + (rb*(k/128) + kb)*2048 + h*1024 + 16*l  (h = 0, 1; l = 0..63)
 *             = the 16 bytes W[rb*16 + l%16][kb*128 + 64*h + 16*(l/16) .. +16)
 *   ws_packed + ((rb*(k/128) + kb)*16 + r)*4
 *             = the 4 scale bytes w_scale[rb*16 + r][kb*4 .. +4)
 *   ws_packed + ceil(n/16)*16*(k/32) + 4*rb
 *             = the range word of row block rb: over its (row, 32-wide block)
 *               pairs holding a nonzero code, the smallest scale byte in bits
 *               0-7 and the largest in bits 8-15 (0xFF and 0 if none)
 * Rows past n are zero codes with scale byte 127. The transform is a one-time
 * re-layout at weight-load time (as FlashInfer's GEMM takes its own swizzled
 * scale layout on the publishing_gemm page); besides the range words it
 * moves bytes only. The GEMM reads the range words to know which row blocks
 * hold nonzero codes under scale bytes outside 3..246, where an e4m3 value
 * times its scale is no longer a BF16 value (see mxgemm_publish).
 * Sizes: ceil(n/16)*16*k bytes, and ceil(n/16)*16*(k/32) plus
 * ceil(ceil(n/16)*4 / 16)*16 bytes; 0 on bad sizes. */
size_t mxgemm_packed_weight_bytes(int32_t n, int32_t k);
size_t mxgemm_packed_scale_bytes(int32_t n, int32_t k);

/* Re-lay row-major W [n, k] (e4m3fn) and w_scale [n, k/32] (E8M0) into the
 * packed layout above. All four pointers are device memory, 16-B aligned;
 * the outputs hold the sizes above. n % 8 == 0, k % 128 == 0. Enqueued on
 * `stream`. Errors: MXG_EINVAL, MXG_EALIGN, MXG_EHIP. */
int mxgemm_pack_weight(const uint8_t* w, const uint8_t* w_scale, int32_t n, int32_t k,
                       uint8_t* w_packed, uint8_t* ws_packed, void* stream);

/* The publishing GEMM (publishing_gemm page, module docstring, "GEMM
 * structure"; PublishingLowLatencyBlockscaledGemmKernel.epilog_warp and
 * publish_value):
 *
 *   C[t, n] = sum_k dec(w[n,k]) 2^(w_scale[n,k/32]-127)
 *                   dec(x[t,k]) 2^(x_scale[t,k/32]-127)
 *
 * accumulated in FP32, rounded to BF16 (nearest even), negative zero cleared,
 * and stored as [m, n] row-major BF16 into bytes [0, 2mn) of slot mb->rank of
 * generation state[NEXT], in 16-byte packs of eight consecutive columns of one
 * token (even column in the low half of each word). One thread then sets
 * state[ACTIVE] = that generation.
 *
 *   w        device, W [n, k] e4m3fn in the packed layout (mxgemm_pack_weight),
 *            16-B aligned
 *   w_scale  device, its E8M0 scales in the packed layout, 16-B aligned
 *   x        device, [m, k] e4m3fn bytes, row-major, 16-B aligned
 *   x_scale  device, [m, k/32] E8M0 bytes, row-major, 16-B aligned
 *   m        activation rows, 1..8
 *   n, k     n % 8 == 0, k % 128 == 0, k % (128 * split_k) == 0
 *   split_k  1, 2, 4 or 8: K is cut into split_k slices; the workgroups of one
 *            output tile exchange FP32 partials through (value, epoch) pairs
 *            in `workspace` and each reduces its share of the tile's packs,
 *            summing the slices in ascending K order.
 *   workspace, workspace_bytes  device, at least mxgemm_workspace_bytes(),
 *            armed by mxgemm_workspace_init; may be NULL/0 when split_k == 1.
 *            One call at a time per workspace.
 *   c_out    device or NULL: [m, n] BF16 as rounded, before the negative-zero
 *            clearing (the plain output of the linear), 16-B aligned.
 *
 * Every publish must be followed by exactly one mailbox_collect of 2*m*n
 * bytes before the next publish into the same mailbox (publishing_gemm page,
 * PublishingMxfp8Linear.precompile: a publish without its consumer would
 * desynchronize the mailbox). Errors: MXG_EINVAL, MXG_EALIGN, MXG_ECAPACITY
 * (2mn > capacity), MXG_EWORKSPACE, MXG_EUNSUPPORTED (the split-K grid cannot
 * be co-resident on this device), MXG_EHIP.
 *
 * Every scale byte 0..254 is taken (255 is the E8M0 NaN). Inside 3..246 each
 * operand is converted with its scale to an exact BF16 value and contracted
 * in BF16 with FP32 accumulation. A 16-row block of W whose range word
 * reaches outside 3..246 but spans at most 243 binades (say scale bytes
 * 0..240, or 20..254) is converted with every scale byte moved by one shift
 * s into 3..246 (exact), and its FP32 partial sums are multiplied by 2^-s
 * once after the K loop. A workgroup whose W rows span more than that, or
 * whose x slice holds a nonzero 32-wide block under a scale byte outside
 * 3..246 (for BF16 x: a block quantized to scale byte 247 or more, the only
 * quantized blocks whose values leave BF16), runs an exact path instead: the
 * MFMA contracts the codes themselves, one 32-wide scale block at a time,
 * and each block's FP32 sum is multiplied by 2^(sW + sX - 254). All paths
 * keep FP32 subnormals; a result or partial sum beyond the FP32 range is
 * infinite or NaN on any, as FP32 accumulation gives.
 *
 * Failure: a split-K poll that gives up (after mb->spin_limit polls) sets
 * MXG_ERR_SPLITK_SPIN in the workspace's ERROR word and leaves its packs
 * unpublished (c_out unwritten there), and every later call on that
 * workspace reads the bit and publishes nothing, so the collect that follows
 * times out (MXG_ERR_COLLECT_SPIN) instead of returning sums of pairs that may
 * be stale. Any MXG_ERR_* bit means: arm the workspace (mxgemm_workspace_init)
 * and the mailbox (mailbox_init) again.
 *
 * The kernel variant (rows per workgroup, waves, W ring depth, whether x is
 * staged in LDS as BF16) is chosen from m, n, k, split_k and the device. Ring
 * depth and x staging leave the result bits unchanged; the number of waves
 * along K sets the FP32 summation order, so variants that differ there agree
 * to rounding, not bit for bit. For measurement and tests mxgemm_tile runs
 * the same GEMM with a chosen variant; the library reads no environment.
 *
 * Host state: the library keeps no configuration between calls. The poll
 * limit travels in the caller's mxg_mailbox; mxgemm, which has none, polls
 * its split-K pairs up to MXG_DEFAULT_SPIN_LIMIT times. What the library does
 * keep are memos of device queries (the default tile per shape and device,
 * the resident-workgroup counts, the no-allocation scratch's device address),
 * which change no result. */
int mxgemm_publish(const mxg_mailbox* mb, const uint8_t* w, const uint8_t* w_scale,
                   const uint8_t* x, const uint8_t* x_scale, int32_t m, int32_t n,
                   int32_t k, int32_t split_k, void* workspace,
                   size_t workspace_bytes, uint16_t* c_out, void* stream);

/* mxgemm_publish for measurement: identical arguments and effects, plus two
 * hipEvent_t (as void*, both required) that HIP records around the GEMM
 * kernel's own execution (hipExtLaunchKernel), so hipEventElapsedTime gives
 * the kernel's duration without launch gaps. Not capturable into a graph.
 * Errors: those of mxgemm_publish; MXG_EINVAL if an event is NULL. */
int mxgemm_publish_timed(const mxg_mailbox* mb, const uint8_t* w, const uint8_t* w_scale,
                         const uint8_t* x, const uint8_t* x_scale, int32_t m, int32_t n,
                         int32_t k, int32_t split_k, void* workspace, size_t workspace_bytes,
                         uint16_t* c_out, void* stream, void* ev_start, void* ev_stop);

/* mxgemm_publish for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, effects and errors as mxgemm_publish, without the
 * workspace: with split_k > 1 the (value, tag) pairs and epoch words live in
 * a library-held device array, one per GPU, held until the process ends,
 * whose pair region is MXG_NOALLOC_PAIR_BYTES (4 MiB); shapes whose
 * mxgemm_workspace_bytes exceed MXG_WS_HEADER_BYTES + MXG_WS_FLAG_BYTES +
 * MXG_NOALLOC_PAIR_BYTES (split_k * ceil(n/8)*8 > 65536) are rejected with
 * MXG_EWORKSPACE before anything is enqueued. The call allocates nothing and
 * the array needs no arming: it starts zero-filled, which the kernel reads
 * as an armed workspace. Every call on a GPU shares that GPU's array and
 * leaves its contents for the next call, so calls that overlap on one GPU (on
 * different streams, or with a mxgemm_publish_noalloc of another mailbox in
 * flight) race and must not be issued; one stream in order is the contract.
 * A split-K poll that gives up sets MXG_ERR_SPLITK_SPIN in the array's own
 * header, which no caller can read or clear. split_k == 1 uses no array and
 * is mxgemm_publish itself. */
#define MXG_NOALLOC_PAIR_BYTES (4u << 20)
int mxgemm_publish_noalloc(const mxg_mailbox* mb, const uint8_t* w, const uint8_t* w_scale,
                           const uint8_t* x, const uint8_t* x_scale, int32_t m, int32_t n,
                           int32_t k, int32_t split_k, uint16_t* c_out, void* stream);

/* mxgemm_publish with the activation in BF16, quantized inside the GEMM
 * (the MXFP8 activation the publishing_gemm page's PublishingMxfp8Linear
 * takes is a QuantizedActivation whose original dtype is BF16; the quantizer
 * itself is not printed). Each workgroup quantizes the K slice of x it
 * needs while its first W loads are in flight: per row and 32 consecutive K,
 * e = the smallest integer with max|x| <= 448 * 2^e, clamped to [-127, 127]
 * (an all-zero block: -127), scale byte e + 127, and each element the
 * e4m3fn value nearest to x / 2^e (ties to even, sign kept). A block holding
 * an infinity or NaN gets scale byte 0xFF and codes 0x7F | sign. The product
 * then is mxgemm_publish's on those codes and scales.
 *   x            device [m, k] BF16 row-major, 16-B aligned.
 *   x_q_out, x_scale_out  both NULL, or device buffers of m*k and m*k/32
 *                bytes (x_q_out 16-B aligned) that receive the quantized
 *                activation (written by the workgroups of the first tile).
 * Other arguments, effects and errors as mxgemm_publish. */
int mxgemm_publish_bf16(const mxg_mailbox* mb, const uint8_t* w, const uint8_t* w_scale,
                        const uint16_t* x, int32_t m, int32_t n, int32_t k, int32_t split_k,
                        void* workspace, size_t workspace_bytes, uint16_t* c_out,
                        uint8_t* x_q_out, uint8_t* x_scale_out, void* stream);

/* The plain GEMM without the publish: mxgemm_publish's product rounded to
 * BF16 into `c_out` (required, [m, n], 16-B aligned), no mailbox touched.
 * It is the first half of the unfused path the publishing_gemm page's
 * module docstring describes (the GEMM writes its output, then a publish
 * kernel reads it back into the mailbox; here mailbox_publish). Other
 * arguments and errors as mxgemm_publish (no MXG_ECAPACITY). */
int mxgemm(const uint8_t* w, const uint8_t* w_scale, const uint8_t* x, const uint8_t* x_scale,
           int32_t m, int32_t n, int32_t k, int32_t split_k, void* workspace,
           size_t workspace_bytes, uint16_t* c_out, void* stream);

/* For tests and measurement, not for callers of the method: the GEMM of
 * mxgemm_publish (mb and x, x_scale given), mxgemm_publish_bf16 (mb and
 * x_bf16 given) or mxgemm (mb null, c_out required) run with a chosen
 * kernel variant instead of the default one. `tile` is "fp8" (the default
 * tile, the x slice kept as FP8 codes in LDS) or "rb,wn,wk,depth[,xr[,x16]]"
 * (16*rb*wn-row tiles of wn*wk waves with `depth` K blocks of W in flight,
 * xr staging rounds, x16 the BF16 x stage; see the variant table in
 * gemm_kernel.h). Results are the same function of the inputs as with the
 * default variant, within the stated tolerance; sum order may differ. The
 * library reads no environment and keeps no override between calls: the
 * variant applies to this call only. Errors: those of the form called, and
 * MXG_EUNSUPPORTED when the variant is not built or does not fit. */
int mxgemm_tile(const char* tile, const mxg_mailbox* mb, const uint8_t* w,
                const uint8_t* w_scale, const uint8_t* x, const uint8_t* x_scale,
                const uint16_t* x_bf16, int32_t m, int32_t n, int32_t k, int32_t split_k,
                void* workspace, size_t workspace_bytes, uint16_t* c_out, uint8_t* x_q_out,
                uint8_t* x_scale_out, void* stream);

/* Stand-alone activation quantizer, the rule of mxgemm_publish_bf16:
 * [rows, k] BF16 `x` (device, 16-B aligned) -> e4m3fn codes `x_q` ([rows,
 * k], 16-B aligned) and E8M0 scales `x_scale` ([rows, k/32]). The unfused
 * form of the quantizing step. Errors: MXG_EINVAL (null, rows < 1, k not a
 * positive multiple of 32), MXG_EALIGN, MXG_EHIP. */
int mxfp8_quantize(const uint16_t* x, int32_t rows, int32_t k, uint8_t* x_q, uint8_t* x_scale,
                   void* stream);

/* Unfused publish: copy `nbytes` of BF16 from `src` (device, 16-B aligned)
 * into slot `rank` with negative zero cleared. For the owner's slot
 * (rank == mb->rank) the generation is state[NEXT] and state[ACTIVE] is set;
 * for an emulated peer slot it is state[PEER_GEN + rank], which the call
 * advances (see the state words above), so peers may publish on another
 * stream while the owner's collect polls. Serves as the emulated peers' publish and as the
 * unfused path the fused epilogue must match bit for bit (publishing_gemm
 * page, module docstring: the consumer sees the same bits either way).
 * Errors: MXG_EINVAL, MXG_EALIGN, MXG_ECAPACITY (nbytes outside
 * (0, capacity] or not a multiple of 16), MXG_EHIP. */
int mailbox_publish(const mxg_mailbox* mb, int32_t rank, const void* src,
                    int64_t nbytes, void* stream);

/* Word publish: mailbox_publish for payloads of arbitrary 32-bit words (the
 * all-gather's input; all_gather page, module docstring, step 1): each word
 * equal to the sentinel 0x80000000 is written as 0, every other word as it
 * is. Serves as the emulated peers' publish for mailbox_all_gather and as its
 * unfused counterpart. Arguments and errors as mailbox_publish. */
int mailbox_publish_words(const mxg_mailbox* mb, int32_t rank, const void* src,
                          int64_t nbytes, void* stream);

/* Fused all-gather of one rank (all_gather page, module docstring, steps
 * 1-3; _AllGatherKernel.kernel), the caller being slot mb->rank: one kernel
 * stores the caller's payload `src` (nbytes, words equal to the sentinel
 * sent as 0) into the caller's slot of generation g = state[NEXT] and, for
 * every rank r, its own included, and pack p < nbytes/16 of generation g,
 * polls the pack until none of its words is the sentinel, writes it to
 * out + (r * nbytes + 16 p), and stores the sentinel back; the last
 * workgroup sets state[NEXT] = (g+1) mod 3. Equivalent to
 * mailbox_publish_words(mb, mb->rank, src) followed by mailbox_collect in
 * one launch. Peers publish with mailbox_publish_words before or during the
 * call. The call
 * takes the place of the caller's publish and collect for that generation:
 * nothing else may publish into the caller's own slot before it. `src` and
 * `out` are device memory, 16-B aligned; `out` holds ranks * nbytes bytes;
 * `src` may be exactly out + rank * nbytes (in place) and must not overlap
 * `out` otherwise. Spin limit and MXG_ERR_COLLECT_SPIN as mailbox_collect.
 * Errors: MXG_EINVAL (null, overlap), MXG_EALIGN, MXG_ECAPACITY, MXG_EHIP. */
int mailbox_all_gather(const mxg_mailbox* mb, const void* src, void* out, int64_t nbytes,
                       void* stream);

/* Collect (all_gather page, module docstring, step 2; _AllGatherKernel.kernel):
 * for every rank r and pack p < nbytes/16 of generation g = state[ACTIVE]
 * (the generation the owner's publish wrote: publishing_gemm page, module
 * docstring, "Ordering", the consumer reads stage_state[1]), poll the pack
 * until none of its four words is the sentinel, write it to
 * out + (r * nbytes + 16 p) (rank-major: [ranks*m, n] for an [m, n]
 * payload), and store the sentinel back; state[NEXT] becomes (g + 1) mod 3
 * (step 3). The owner's publish (mxgemm_publish or mailbox_publish into slot
 * mb->rank) must precede the collect on its stream. A pack still holding a sentinel after
 * mb->spin_limit polls is copied as it is and MXG_ERR_COLLECT_SPIN is set in
 * state[ERROR]. `out` is device memory of ranks * nbytes bytes, 16-B aligned.
 * Errors: MXG_EINVAL, MXG_EALIGN, MXG_ECAPACITY, MXG_EHIP. */
int mailbox_collect(const mxg_mailbox* mb, void* out, int64_t nbytes, void* stream);

/* All-reduce collect: the consumer that sums the ranks' published outputs
 * (publishing_gemm page, module docstring: the boundary all-reduce after the
 * row-parallel GEMM). The pages do not print its internals; this is the plain
 * meaning in FP32. For every pack p < nbytes/16 of generation g =
 * state[ACTIVE], each rank's pack is polled as in mailbox_collect, the eight
 * BF16 values at each position are added in FP32 in ascending rank order,
 * and the sums are rounded once to BF16 (nearest even) into out + 16 p
 * ([m, n] BF16 for an [m, n] payload; a sum can round to negative zero).
 * Every rank's pack is reset to the sentinel and the generation advances as
 * in mailbox_collect; a pack still holding a sentinel after mb->spin_limit polls
 * sets MXG_ERR_COLLECT_SPIN. `out` is device memory of nbytes bytes, 16-B
 * aligned. Errors: MXG_EINVAL, MXG_EALIGN, MXG_ECAPACITY, MXG_EHIP. */
int mailbox_collect_sum(const mxg_mailbox* mb, void* out, int64_t nbytes, void* stream);

/* Measurement aid, not a step of the method: a plain HBM read of `bytes`
 * (a positive multiple of 16, at most 2^40) from device memory `src` (16-B
 * aligned), nothing else. It measures what this device's HBM delivers to a
 * pure read stream of that size, the context for the GEMM's roofline
 * fraction. Each MXG_STREAM_CHUNK_BYTES chunk i (the last one may be short)
 * is read by one workgroup, which stores the XOR of the chunk's
 * little-endian 32-bit words into sink[i]; `sink` is device memory of
 * ceil(bytes / MXG_STREAM_CHUNK_BYTES) words. Errors: MXG_EINVAL, MXG_EALIGN,
 * MXG_EHIP. */
#define MXG_STREAM_CHUNK_BYTES 32768
int mxg_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

/* Measurement aid, not a step of the method: the same plain read of `bytes`
 * with the choices a streaming kernel makes exposed, to find what read
 * organisation this device's HBM rewards. threads: 256 or 512 per
 * workgroup; unroll: 4, 8 or 16 16-byte loads per thread in flight;
 * load_kind: 0 global nontemporal, 1 global default policy, 2 raw buffer
 * nontemporal, 3 raw buffer default policy (2 and 3: bytes at most
 * 0x7FFF0000), 4 global straight into LDS (global_load_lds_dwordx4,
 * nontemporal; each lane then reads its 16 bytes back from LDS); workgroups: 0 for one workgroup per MXG_STREAM_CHUNK_BYTES
 * chunk, else that many workgroups, each reading one contiguous range of
 * ceil(bytes/16 / workgroups) 16-byte words (interleave 0) or the chunks
 * g, g + workgroups, ... (interleave 1, needs workgroups > 0). Workgroup g
 * stores the XOR of every little-endian 32-bit word it read into sink[g];
 * `sink` holds one word per workgroup. Errors: MXG_EINVAL, MXG_EALIGN,
 * MXG_EHIP. */
int mxg_stream_read_cfg(const void* src, size_t bytes, uint32_t* sink, int32_t workgroups,
                        int32_t threads, int32_t unroll, int32_t load_kind, int32_t interleave,
                        void* stream);

/* Measurement aid, not a step of the method: C[16][16] = sum over k of
 * A[row][k] * 2^(as[row][k/32] - 127) * B[col][k] * 2^(bs[col][k/32] - 127)
 * for e4m3fn A and B ([16][k] each, row-major, K contiguous) and their E8M0
 * scales ([16][k/32] each), accumulated in FP32 by one wave in 128-wide K
 * steps, into c[row * 16 + col] (FP32, device memory). scaled = 1 uses the
 * block-scaled fp8 MFMA that the publishing_gemm page's MXFP8 linear layer
 * runs (FlashInfer's mm_mxfp8, sf_vec_size 32); on gfx950 that is
 * v_mfma_scale_f32_16x16x128_f8f6f4. scaled = 0 uses this library's GEMM
 * arithmetic: each code times its scale converted to BF16 (exact for scale
 * bytes 3..246), then v_mfma_f32_16x16x32_bf16. It exists so that the
 * accuracy of the two on the same inputs can be compared on the device.
 * k: a positive multiple of 128; all pointers 16-B aligned, scales may be
 * any address. Errors: MXG_EINVAL, MXG_EALIGN, MXG_EHIP. */
int mxg_probe_mfma(const uint8_t* a, const uint8_t* a_scale, const uint8_t* b,
                   const uint8_t* b_scale, int32_t k, int32_t scaled, float* c, void* stream);

/* HIP graph helpers: capture the calls issued on `stream` between begin and
 * end into an executable graph, replay it, destroy it. `exec` is an opaque
 * hipGraphExec_t. Kernels must have been launched once before capture
 * (publishing_gemm page, PublishingMxfp8Linear.precompile: compile before
 * capture). Errors: MXG_EINVAL, MXG_EHIP. */
int mxg_graph_begin(void* stream);
int mxg_graph_end(void* stream, void** exec);
int mxg_graph_launch(void* exec, void* stream);
int mxg_graph_destroy(void* exec);

/* Static string describing a return code. */
const char* mxg_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* MXGEMM_H */
