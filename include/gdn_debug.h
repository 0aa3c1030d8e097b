/*
 * gdn_debug.h -- the index checks of the debug build of the library.
 *
 * libgdn_debug.so is the library with its prefill kernels (chunk_mfma.hip: the per-chunk prep,
 * the state pass, the combined launches of the pieced split path, the pipelined and the fused
 * kernels) compiled with GDN_DEBUG (and with the test hooks of libgdn_hooks.so, so that tests can
 * pick each route).  Its kernels check the indices they derive -- workgroup to chain, segment
 * and piece bounds, workspace chunks, token rows of the output -- and a failed check sets one bit
 * in a per-device flags word instead of trapping; every checked access is also clamped or guarded
 * by the surrounding code, so the kernel still ends normally.  It is a testing aid for callers
 * and for this library's own tests; libgdn.so neither checks nor exports this call.
 */
#ifndef GDN_DEBUG_H
#define GDN_DEBUG_H

#ifdef __cplusplus
extern "C" {
#endif

/*
 * gdn_debug_take_flags -- waits for the current device (hipDeviceSynchronize), returns the checks
 * that failed there since the previous call and clears them.  Bits: 0 prep unit, 1 state-pass
 * chain, 2 state-pass segment or piece, 3 state-pass workspace chunk, 4 state-pass output token,
 * 5 pipelined-kernel chain and tokens, 6 combined launch of the pieced split path, 7 fused-kernel
 * chain.  0 means every check held; 0xffffffff means the flags could not be read (no device, or
 * a HIP error).  Only in libgdn_debug.so.
 */
unsigned int gdn_debug_take_flags(void);

/*
 * gdn_debug_self_test -- enqueues, on the null stream of the current device, one tiny kernel
 * whose only work is a check that fails at `bit` (0..31), so that the next gdn_debug_take_flags
 * returns that bit: a test of the flags' path itself.  Returns 0, or -1 for a bit outside 0..31
 * or a launch error.  Only in libgdn_debug.so.
 */
int gdn_debug_self_test(int bit);

#ifdef __cplusplus
}
#endif

#endif /* GDN_DEBUG_H */
