/*
 * sai_profile.h -- profiling aid of the paged lightning-indexer library
 * (not an operation of the pages; nothing on the indexer's path needs it).
 *
 * sai_time_next_launch arms a pair of events (created by the caller with
 * hipEventCreate*) for the next kernel that the calling thread launches
 * through any entry point of sai.h: that launch carries them in its own
 * dispatch, so hipEventElapsedTime(start, stop) is the kernel's execution
 * time without the marker packets a separate hipEventRecord adds to the
 * stream.  The pair is used once; entry points that launch several kernels
 * time the first.  Both NULL disarms.
 *
 * State: the armed pair is kept per thread (thread_local) until that
 * thread's next launch; it is the only state the library keeps between
 * calls, and it changes no result.  No device work.
 *
 * Returns SAI_OK, or SAI_EINVAL if exactly one event is NULL.
 *
 * sai_time_span arms a pair that spans several kernels: the next launch
 * carries start, and every launch until the thread disarms the span (both
 * NULL, here or through sai_time_next_launch) carries stop, so after
 * arm -> calls -> disarm, hipEventElapsedTime(start, stop) runs from the
 * first kernel's start to the last kernel's end, gaps between them
 * included (the way to time an entry point that launches several
 * kernels).  Same per-thread state and return codes as above.
 */
#ifndef SAI_PROFILE_H
#define SAI_PROFILE_H

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

int sai_time_next_launch(hipEvent_t start, hipEvent_t stop);
int sai_time_span(hipEvent_t start, hipEvent_t stop);

#ifdef __cplusplus
}
#endif
#endif /* SAI_PROFILE_H */
