/*
 * sqattn checking build: exported by libsqattn_debug.so only (built beside
 * libsqattn.so with -DSQATTN_DEBUG).  That library is the same C-ABI
 * (include/sqattn.h) with two differences in the attention kernels: every
 * wait in front of a work-group barrier drains all loads in flight (the
 * release build waits only for the loads the next phase reads), and the
 * kernels check their K/V tile indices, the last K row they read and the
 * block-sparse tile list length, setting one bit of a device word per failed
 * check.  Its outputs must equal the release build's bit for bit; a
 * difference points at a missing wait.  For tests, not for production use.
 */
#ifndef SQATTN_DEBUG_H
#define SQATTN_DEBUG_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The current device's violation word since the previous call, then reset
 * to 0 (synchronizes the device).  Bits: 0 K tile index out of [0, nt),
 * 1 V tile index out of [0, nt), 2 a K tile with no row before N, 3 a
 * block-sparse tile list longer than its LDS space, 4 a tile of the
 * exact-max second pass out of range.  0xFFFFFFFF: the word could not be
 * read. */
uint32_t sqattn_debug_violations(void);

#ifdef __cplusplus
}
#endif

#endif /* SQATTN_DEBUG_H */
