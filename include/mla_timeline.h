/* Timeline stamps of the decode kernels: present only in libmla_decode_timeline.so, the
 * same sources built with MLA_TIMELINE defined (mla_split_kv_decode_amd/build.py,
 * build_timeline).  Wave 0 of every workgroup writes the device's 100 MHz real-time clock
 * (s_memrealtime) at fixed points; a workgroup that runs several pieces keeps those of its
 * last piece; slots a workgroup never reaches stay as they were (clear them first).  The
 * probes wait for the wave's outstanding scalar loads, which is why the entry stamp is the
 * kernel's first statement and none sits between entry and a piece's first copies.
 *
 * Partial kernel, uint64 [4096 workgroups][8 slots] (blocks past 4096 do not stamp):
 *   0 entry; 1 the piece's first page copies issued; 2 the queries read out of the staging
 *   tile; 3, 4 pages 0 and 1 landed in every wave (page pairs 0 and 1 for the FP8 two-row
 *   kernels); 5 epilogue: row denominators exchanged; 6 partial answers issued; 7 partial
 *   answers stored (the stamping build waits for its stores here).
 * Merge kernels, uint64 [16384 workgroups][4 slots]:
 *   0 entry; 1 the row's LSE maximum known; 2 the partial answers consumed (column-chunk
 *   merge only); 3 end.
 */
#ifndef MLA_TIMELINE_H
#define MLA_TIMELINE_H

#ifdef __cplusplus
extern "C" {
#endif

/* Copy the stamps to host arrays of 4096 * 8 and 16384 * 4 uint64.  0 on success. */
int mla_timeline_read(unsigned long long* partial, unsigned long long* merge);
/* Zero every stamp (synchronous).  0 on success. */
int mla_timeline_clear(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_TIMELINE_H */
