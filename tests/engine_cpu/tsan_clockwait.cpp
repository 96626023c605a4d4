// Linked into the ThreadSanitizer build of engine_check only.
//
// libstdc++ implements std::condition_variable::wait_for / wait_until on the
// steady clock with pthread_cond_clockwait, which the ThreadSanitizer
// runtime of GCC 11 does not intercept: it then never sees the mutex being
// released inside the wait, and the next thread to take that mutex is
// reported as a double lock, followed by data races under the mutex (a
// correct ten-line program shows the same).  This definition takes the call
// in the test binary and waits with pthread_cond_timedwait, which the
// runtime does intercept, on the same deadline moved to CLOCK_REALTIME.
#include <pthread.h>
#include <time.h>

extern "C" int pthread_cond_clockwait(pthread_cond_t* cond, pthread_mutex_t* mutex, clockid_t clock,
                                      const struct timespec* abstime) {
  timespec now_c, now_r;
  clock_gettime(clock, &now_c);
  clock_gettime(CLOCK_REALTIME, &now_r);
  long long ns = (static_cast<long long>(abstime->tv_sec) - now_c.tv_sec) * 1000000000LL +
                 (abstime->tv_nsec - now_c.tv_nsec);
  if (ns < 0) ns = 0;
  timespec deadline;
  const long long total = static_cast<long long>(now_r.tv_nsec) + ns % 1000000000LL;
  deadline.tv_sec = now_r.tv_sec + static_cast<time_t>(ns / 1000000000LL + total / 1000000000LL);
  deadline.tv_nsec = static_cast<long>(total % 1000000000LL);
  return pthread_cond_timedwait(cond, mutex, &deadline);
}
